// Block level of the hierarchical indexer: block summaries, block scores
// and the top-m block choice.
//
// Block summaries follow the HISA explainer, section 1.2.1 (fixed-size
// blocks, mean pooling) and the HISA news article ("block-level coarse
// filter"); block scores use the indexer's own dot product against the
// block features (same sources); the block choice keeps the first block and
// the query's own block and fills the rest with the best-scoring complete
// blocks before it (HISA explainer 1.2.1 item 3, HISA news article).
#include <type_traits>

#include "common.hpp"
#include "internal.h"
#include "select.hpp"

namespace hisa {

// ------------------------------------------------------------------ summary
// One workgroup per (block, sequence). Threads read 16-byte column groups of
// the block's rows (coalesced), sum in fp32, reduce the row-parallel partial
// sums through LDS, optionally project with proj (fp32, fixed order), and
// write the mean plus the exact bf16 hi/mid/lo split of the (projected) sum.
template <int D>
// Row c = first_row + blockIdx.x of sequence blockIdx.y; tables hold n_rows
// rows per sequence.
__global__ __launch_bounds__(256) void block_summary_kernel(
    const uint16_t* __restrict__ kidx, int64_t ksb, int64_t kst, int L, int B, int n_rows,
    int first_row, const uint16_t* __restrict__ proj, float* __restrict__ summary,
    uint16_t* __restrict__ split) {
  constexpr int TPR = D / 8;      // threads per row (8 columns each)
  constexpr int RP = 256 / TPR;   // rows summed in parallel
  __shared__ float part[RP][D + 1];
  __shared__ float sums[D];
  const int c = first_row + blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int col0 = (tid % TPR) * 8, r0 = tid / TPR;
  const int j0 = c * B, j1 = min(L, j0 + B);
  const uint16_t* base = kidx + b * ksb;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
  for (int j = j0 + r0; j < j1; j += RP) {
    const uint4 w = *reinterpret_cast<const uint4*>(base + j * kst + col0);
    acc[0] += bf16_lo(w.x); acc[1] += bf16_hi(w.x);
    acc[2] += bf16_lo(w.y); acc[3] += bf16_hi(w.y);
    acc[4] += bf16_lo(w.z); acc[5] += bf16_hi(w.z);
    acc[6] += bf16_lo(w.w); acc[7] += bf16_hi(w.w);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[r0][col0 + e] = acc[e];
  __syncthreads();
  float s = 0.0f;
  if (tid < D) {
    for (int r = 0; r < RP; ++r) s += part[r][tid];
    sums[tid] = s;
  }
  __syncthreads();
  if (tid < D) {
    if (proj != nullptr) {
      const uint16_t* wr = proj + tid * D;
      float p = 0.0f;
      for (int i = 0; i < D; i += 8) {
        const uint4 w = *reinterpret_cast<const uint4*>(wr + i);
        p = fmaf(bf16_lo(w.x), sums[i + 0], p); p = fmaf(bf16_hi(w.x), sums[i + 1], p);
        p = fmaf(bf16_lo(w.y), sums[i + 2], p); p = fmaf(bf16_hi(w.y), sums[i + 3], p);
        p = fmaf(bf16_lo(w.z), sums[i + 4], p); p = fmaf(bf16_hi(w.z), sums[i + 5], p);
        p = fmaf(bf16_lo(w.w), sums[i + 6], p); p = fmaf(bf16_hi(w.w), sums[i + 7], p);
      }
      s = p;
    }
    const int64_t row = static_cast<int64_t>(b) * n_rows + c;
    if (summary != nullptr) summary[row * D + tid] = s / static_cast<float>(j1 - j0);
    if (split != nullptr) {
      // hi + mid + lo == s exactly: each remainder is exact (the rounded
      // term lies within a factor of two of the value it is taken from) and
      // the last remainder has at most 8 significant bits.
      const uint16_t hi = f32_to_bf16(s);
      const float r1 = s - bf16_to_f32(hi);
      const uint16_t mid = f32_to_bf16(r1);
      const float r2 = r1 - bf16_to_f32(mid);
      const uint16_t lo = f32_to_bf16(r2);
      uint16_t* o = split + row * 3 * D;
      o[tid] = hi;
      o[D + tid] = mid;
      o[2 * D + tid] = lo;
    }
  }
}

hipError_t launch_block_summary(const uint16_t* kidx, Str3 ks, int batch, int L, int d, int B,
                                const uint16_t* proj, float* summary, uint16_t* split,
                                int n_rows_cap, int first_row, hipStream_t s) {
  const int n_rows = (L + B - 1) / B;
  dim3 grid(n_rows - first_row, batch);
  if (d == 64)
    hipLaunchKernelGGL(block_summary_kernel<64>, grid, dim3(256), 0, s, kidx, ks.b, ks.t, L, B,
                       n_rows_cap, first_row, proj, summary, split);
  else
    hipLaunchKernelGGL(block_summary_kernel<128>, grid, dim3(256), 0, s, kidx, ks.b, ks.t, L, B,
                       n_rows_cap, first_row, proj, summary, split);
  return hipGetLastError();
}

// ------------------------------------------------------------------ scores
// Tile: 64 queries x 64 blocks per workgroup, 16 queries per wave. The
// contraction (hi + mid + lo) . q runs on the bf16 matrix cores with fp32
// accumulation (K = 3*D); for integer-valued keys every partial sum is an
// integer below 2^24, so the score is exact, then scaled by 1/B (exact for
// a power-of-two B). The summaries are the A operand (rows = blocks) and the
// queries the B operand, so each lane ends with four consecutive blocks of
// one query and stores them with one 16-byte write. The twelve fragments of
// a 16-block step are loaded together.
template <int D>
__global__ __launch_bounds__(256) void block_score_kernel(
    const uint16_t* __restrict__ qidx, int64_t qsb, int64_t qst, const int32_t* __restrict__ q_pos,
    int nq, const uint16_t* __restrict__ split, int n_rows, int B, float invB,
    float* __restrict__ out) {
  constexpr int KS = D / 32;
  const int wave = threadIdx.x / kWave, lane = lane_id();
  const int b = blockIdx.z;
  // query tiles vary fastest: consecutive workgroups go to the XCDs in turn,
  // so each XCD gets every eighth query tile with all its block tiles, and
  // the causal work (more blocks for later queries) is spread evenly
  const int q0 = blockIdx.x * 64 + wave * 16;
  const int c0 = blockIdx.y * 64;
  const int g = lane / 16, r16 = lane % 16;
  if (q0 >= nq) return;
  // this lane's query (column r16 of the products) and its local block
  const int qq = q0 + r16;
  const int qc = min(qq, nq - 1);
  const int bt = qq < nq ? min(max(q_pos[static_cast<int64_t>(b) * nq + qc], 0), n_rows * B - 1) / B
                         : -1;
  const int btmax = static_cast<int>(wave_max(static_cast<float>(bt)));
  // B fragments: the query row of this lane, 8 values per k step
  const uint16_t* qrow = qidx + b * qsb + static_cast<int64_t>(qc) * qst + 8 * g;
  bf16x8 qf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) qf[s] = as_bf16x8(*reinterpret_cast<const uint4*>(qrow + 32 * s));
  float* orow = out + (static_cast<int64_t>(b) * nq + qc) * n_rows;
  const bool vec = (n_rows & 3) == 0;
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int cb = c0 + nt * 16;
    if (cb >= n_rows) break;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    if (cb < btmax) {
      // A fragments: block cb + r16 of the summary table (hi, mid, lo terms)
      const int cc = min(cb + r16, n_rows - 1);
      const uint16_t* srow = split + (static_cast<int64_t>(b) * n_rows + cc) * 3 * D + 8 * g;
      uint4 sf[3 * KS];
#pragma unroll
      for (int x = 0; x < 3 * KS; ++x)
        sf[x] = *reinterpret_cast<const uint4*>(srow + (x / KS) * D + 32 * (x % KS));
      __builtin_amdgcn_sched_barrier(0);  // all of them in flight before the first product
#pragma unroll
      for (int x = 0; x < 3 * KS; ++x) acc = mfma16(as_bf16x8(sf[x]), qf[x % KS], acc);
    }
    // lane: blocks cb + 4g + (0..3) of query qq
    if (qq < nq) {
      const int c = cb + 4 * g;
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = c + r < bt ? acc[r] * invB : -INFINITY;
      if (vec && c + 3 < n_rows) {
        *reinterpret_cast<float4*>(orow + c) = make_float4(v[0], v[1], v[2], v[3]);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (c + r < n_rows) orow[c + r] = v[r];
      }
    }
  }
}

hipError_t launch_block_score(const uint16_t* qidx, Str3 qs, const int32_t* q_pos, int batch,
                              int nq, const uint16_t* split, int n_rows, int d, int B,
                              float* scores, hipStream_t s) {
  dim3 grid((nq + 63) / 64, (n_rows + 63) / 64, batch);
  const float invB = 1.0f / static_cast<float>(B);
  if (d == 64)
    hipLaunchKernelGGL(block_score_kernel<64>, grid, dim3(256), 0, s, qidx, qs.b, qs.t, q_pos, nq,
                       split, n_rows, B, invB, scores);
  else
    hipLaunchKernelGGL(block_score_kernel<128>, grid, dim3(256), 0, s, qidx, qs.b, qs.t, q_pos,
                       nq, split, n_rows, B, invB, scores);
  return hipGetLastError();
}

// ------------------------------------------------------------------ top-m
// One workgroup per query. Candidates are blocks 1 .. b-1 (position p is
// block p+1); the first block and the local block b are added around the
// free picks, which keeps the output ascending.
template <int NT, int ITEMS, bool CACHED>
__global__ __launch_bounds__(NT) void select_blocks_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ q_pos, int nq, int n_rows,
    int B, int m, int32_t* __restrict__ block_idx) {
  constexpr int NB = NT >= 256 ? 2048 : 256;
  __shared__ SelectLds<NT, NB> sh;
  const int64_t qi = static_cast<int64_t>(blockIdx.y) * nq + blockIdx.x;
  const float* row = scores + qi * n_rows;
  int32_t* out = block_idx + qi * m;
  const int t = min(max(q_pos[qi], 0), n_rows * B - 1);
  const int bt = t / B;
  const int n = max(bt - 1, 0);
  const int free_slots = m - (bt == 0 ? 1 : 2);
  if (n <= free_slots) {
    for (int i = threadIdx.x; i < m; i += NT) out[i] = i <= bt ? i : -1;
    return;
  }
  constexpr int CH = NT * ITEMS;
  const int nchunks = (n + CH - 1) / CH;
  float vals[CACHED ? ITEMS : 1];
  if constexpr (CACHED) {
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const int p = threadIdx.x * ITEMS + i;
      vals[i] = p < n ? row[1 + p] : 0.0f;
    }
  }
  auto get = [&](int c, int i, float& v) -> bool {
    const int p = c * CH + threadIdx.x * ITEMS + i;
    if (p >= n) return false;
    if constexpr (CACHED) v = vals[i]; else v = row[1 + p];
    return true;
  };
  const Threshold th = select_threshold<NT, ITEMS, NB>(get, nchunks, free_slots, sh);
  uint32_t kept = 0, ties = 0;
  for (int c = 0; c < nchunks; ++c) {
    select_compact<NT, ITEMS, NB>(get, c, th, kept, ties, sh, [&](uint32_t pos, int i, float) {
      out[1 + pos] = c * CH + threadIdx.x * ITEMS + i + 1;
    });
  }
  if (threadIdx.x == 0) {
    out[0] = 0;
    out[1 + free_slots] = bt;
  }
}

// The same selection without workgroup barriers. A wave holds its candidates
// item-major (item i of lane l is position base + 64i + l) as order-preserving
// 32-bit keys (0, below every finite score's key, for no candidate), finds the
// K-th largest by bisection on the key (each step one comparison per item,
// counted on the scalar unit from the comparison's lane mask), and writes the kept ones
// in position order with ballots: those above the threshold and the first
// `need` equal to it. With W > 1 waves, wave w keeps the best K of its slice
// of 64*IT candidates (each of the K best overall is among the K best of its
// slice under the same order), the kept keys and positions meet in LDS in
// position order, and wave 0 selects the best K of those.
struct WaveSel {
  uint32_t T;     // threshold key: keys > T kept
  uint32_t need;  // plus the first `need` keys == T
};

template <int IT>
__device__ __forceinline__ WaveSel wave_select(const uint32_t (&key)[IT], uint32_t okm,
                                               uint32_t K) {
  // the smallest and largest key of the candidates, on the keys themselves
  // (their order is the scores' order); with no candidate lo > hi
  uint32_t mn = 0xffffffffu, mx = 0u;
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const bool ok = ((okm >> i) & 1u) && key[i] != 0u;
    mn = min(mn, ok ? key[i] : 0xffffffffu);
    mx = max(mx, ok ? key[i] : 0u);
  }
  uint32_t lo = wave_min_u32(mn), hi = wave_max_u32(mx);
  // the largest key x with count(key >= x) >= K (keys of no candidate are 0 < lo)
  while (lo < hi) {
    const uint32_t mid = lo + ((hi - lo + 1u) >> 1);
    uint32_t c = 0;
#pragma unroll
    for (int i = 0; i < IT; ++i) c += static_cast<uint32_t>(__popcll(__ballot(key[i] >= mid)));
    if (c == K) {
      // exactly the K largest keys are >= mid: the K-th largest is their
      // minimum (usually reached after a third of the steps, once mid falls
      // in the gap between the K-th and the next key)
      uint32_t m = 0xffffffffu;
#pragma unroll
      for (int i = 0; i < IT; ++i) m = key[i] >= mid ? min(m, key[i]) : m;
      lo = hi = wave_min_u32(m);
      break;
    }
    if (c > K) lo = mid; else hi = mid - 1u;
  }
  uint32_t gt = 0;
#pragma unroll
  for (int i = 0; i < IT; ++i) gt += static_cast<uint32_t>(__popcll(__ballot(key[i] > lo)));
  return WaveSel{lo, K - gt};
}

template <int IT, class Emit>
__device__ __forceinline__ void wave_compact(const uint32_t (&key)[IT], uint32_t okm,
                                             const WaveSel s, Emit emit) {
  uint32_t kept = 0, ties = 0;
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const bool ok = (okm >> i) & 1u;
    const bool eq = ok && key[i] == s.T;
    const uint64_t em = __ballot(eq);
    const bool keep = ok && (key[i] > s.T || (eq && ties + lanes_below(em) < s.need));
    const uint64_t km = __ballot(keep);
    if (keep) emit(i, kept + lanes_below(km));
    ties += static_cast<uint32_t>(__popcll(em));
    kept += static_cast<uint32_t>(__popcll(km));
  }
}

// Top K <= 64 of a wave's items with fewer vector instructions: the K-th
// largest of the 64 lane maxima is a lower bound of the K-th largest item
// (K lanes hold an item at least that large), so only the items at or above
// it can be kept. For spread scores they are a few dozen: they are moved to
// LDS in position order (lkey/lpos, kSelSmall entries) and the exact
// selection runs on two items per lane. More than kSelSmall of them (mass
// ties) takes the direct path. emit(rank, position) gets the kept positions
// in ascending order, rank 0 .. K-1.
constexpr int kSelSmall = 128;

template <int IT, class Emit>
__device__ __forceinline__ void wave_topk(const uint32_t (&key)[IT], uint32_t okm, uint32_t K,
                                          uint32_t* lkey, int* lpos, Emit emit) {
  const int l = lane_id();
  if constexpr (IT >= 4) {
    if (K <= 64) {
      uint32_t lm = 0;
#pragma unroll
      for (int i = 0; i < IT; ++i) lm = (okm >> i) & 1u ? max(lm, key[i]) : lm;
      const uint32_t lk[1] = {lm};
      const uint32_t t1 = wave_select(lk, 1u, K).T;
      uint32_t c = 0;
#pragma unroll
      for (int i = 0; i < IT; ++i)
        c += static_cast<uint32_t>(__popcll(__ballot(((okm >> i) & 1u) && key[i] >= t1)));
      if (c <= kSelSmall) {
        uint32_t base = 0;
#pragma unroll
        for (int i = 0; i < IT; ++i) {
          const bool keep = ((okm >> i) & 1u) && key[i] >= t1;
          const uint64_t km = __ballot(keep);
          if (keep) {
            const uint32_t e = base + lanes_below(km);
            lkey[e] = key[i];
            lpos[e] = 64 * i + l;
          }
          base += static_cast<uint32_t>(__popcll(km));
        }
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
        uint32_t k2[kSelSmall / 64];
        uint32_t ok2 = 0;
#pragma unroll
        for (int i = 0; i < kSelSmall / 64; ++i) {
          const uint32_t e = 64 * i + l;
          k2[i] = e < c ? lkey[e] : 0u;
          ok2 |= e < c ? (1u << i) : 0u;
        }
        const WaveSel sel = wave_select(k2, ok2, K);
        wave_compact(k2, ok2, sel, [&](int i, uint32_t pos) { emit(pos, lpos[64 * i + l]); });
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
        return;
      }
    }
  }
  const WaveSel sel = wave_select(key, okm, K);
  wave_compact(key, okm, sel, [&](int i, uint32_t pos) { emit(pos, 64 * i + l); });
}

constexpr int kSelUnion = 1024;  // LDS entries for the waves' kept candidates

// TOPK (W > 1): each wave, and wave 0 over the union, uses wave_topk, the
// faster choice for a few queries keeping at most 32 blocks; many queries
// fill the chip better with the plain wave_select.
template <int W, int IT, bool TOPK = false>
__global__ __launch_bounds__(64 * W) void select_blocks_wave_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ q_pos, int nq, int n_rows,
    int B, int m, int32_t* __restrict__ block_idx) {
  constexpr int S = 64 * IT;  // candidates per wave
  constexpr int CAP = W > 1 ? kSelUnion : kSelSmall;
  __shared__ uint32_t ckey[CAP];
  __shared__ int cpos[CAP];
  __shared__ int ccnt[W];
  // with TOPK: wave_topk's survivors, one slice per wave
  __shared__ uint32_t skey[TOPK ? W : 1][kSelSmall];
  __shared__ int spos[TOPK ? W : 1][kSelSmall];
  const int64_t qi = static_cast<int64_t>(blockIdx.y) * nq + blockIdx.x;
  const float* row = scores + qi * n_rows;
  int32_t* out = block_idx + qi * m;
  const int t = min(max(q_pos[qi], 0), n_rows * B - 1);
  const int bt = t / B;
  const int n = max(bt - 1, 0);
  const int K = m - (bt == 0 ? 1 : 2);  // free slots
  if (n <= K) {
    for (int i = threadIdx.x; i < m; i += 64 * W) out[i] = i <= bt ? i : -1;
    return;
  }
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), l = lane_id();
  const int base = w * S;
  uint32_t key[IT];
  uint32_t okm = 0;
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const int p = base + 64 * i + l;
    key[i] = p < n ? order_key(row[1 + p]) : 0u;
    okm |= p < n ? (1u << i) : 0u;
  }
  if constexpr (W == 1) {
    if (K > 0)
      wave_topk(key, okm, static_cast<uint32_t>(K), ckey, cpos,
                [&](uint32_t pos, int p) { out[1 + pos] = p + 1; });
  } else {
    const int kw = min(K, max(0, min(S, n - base)));  // kept by this wave
    if (kw > 0) {
      if constexpr (TOPK) {
        // the kept key is read back from the row (it is in cache)
        wave_topk(key, okm, static_cast<uint32_t>(kw), skey[w], spos[w], [&](uint32_t pos, int p) {
          ckey[w * K + pos] = order_key(row[1 + base + p]);
          cpos[w * K + pos] = base + p;
        });
      } else {
        const WaveSel sel = wave_select(key, okm, static_cast<uint32_t>(kw));
        wave_compact(key, okm, sel, [&](int i, uint32_t pos) {
          ckey[w * K + pos] = key[i];
          cpos[w * K + pos] = base + 64 * i + l;
        });
      }
    }
    if (l == 0) ccnt[w] = kw;
    __syncthreads();
    if (w == 0 && K > 0) {
      // entry e = u*K + j is the j-th kept candidate of wave u: position order
      constexpr int IB = CAP / 64;
      uint32_t k2[IB];
      uint32_t ok2 = 0;
#pragma unroll
      for (int i = 0; i < IB; ++i) {
        const int e = 64 * i + l;
        const int u = e / K;
        const bool ok = u < W && e - u * K < ccnt[min(u, W - 1)];
        k2[i] = ok ? ckey[e] : 0u;
        ok2 |= ok ? (1u << i) : 0u;
      }
      if constexpr (TOPK) {
        wave_topk(k2, ok2, static_cast<uint32_t>(K), skey[0], spos[0],
                  [&](uint32_t pos, int e) { out[1 + pos] = cpos[e] + 1; });
      } else {
        const WaveSel sel = wave_select(k2, ok2, static_cast<uint32_t>(K));
        wave_compact(k2, ok2, sel,
                     [&](int i, uint32_t pos) { out[1 + pos] = cpos[64 * i + l] + 1; });
      }
    }
  }
  if (threadIdx.x == 0) {
    out[0] = 0;
    out[1 + K] = bt;
  }
}

hipError_t launch_select_blocks(const float* scores, const int32_t* q_pos, int batch, int nq,
                                int n_rows, int B, int m, int32_t* block_idx, hipStream_t s) {
  dim3 grid(nq, batch);
#define HISA_SW(W_, IT_)                                                                        \
  hipLaunchKernelGGL((select_blocks_wave_kernel<W_, IT_>), grid, dim3(64 * W_), 0, s, scores,   \
                     q_pos, nq, n_rows, B, m, block_idx)
  // The wave select trades latency for throughput: a wave's ~32 dependent
  // bisection steps are slower than the histogram select's few levels when
  // only a few queries run, and faster once many queries fill the chip.
  const bool many = static_cast<int64_t>(batch) * nq >= 1024;
  // candidates are blocks 1 .. n_rows-2 at most
  if (!many) {
    if (n_rows <= 64 * 16)
      hipLaunchKernelGGL((select_blocks_kernel<64, 16, true>), grid, dim3(64), 0, s, scores,
                         q_pos, nq, n_rows, B, m, block_idx);
    // measured: from 6,144 blocks on, with m = 32, 16 waves with wave_topk
    // beat the histogram select (16,384 blocks: 22 vs 32 us); with m = 64
    // and at 4,096 blocks the histogram select stays faster
    else if (n_rows > 4 * 1024 + 2 && n_rows <= 16 * 1024 && m - 2 <= 32)
      hipLaunchKernelGGL((select_blocks_wave_kernel<16, 16, true>), grid, dim3(64 * 16), 0, s,
                         scores, q_pos, nq, n_rows, B, m, block_idx);
    else if (n_rows <= 1024 * 16)
      hipLaunchKernelGGL((select_blocks_kernel<1024, 16, true>), grid, dim3(1024), 0, s, scores,
                         q_pos, nq, n_rows, B, m, block_idx);
    else
      hipLaunchKernelGGL((select_blocks_kernel<1024, 16, false>), grid, dim3(1024), 0, s, scores,
                         q_pos, nq, n_rows, B, m, block_idx);
  } else if (n_rows <= 64 + 2) HISA_SW(1, 1);
  else if (n_rows <= 128 + 2) HISA_SW(1, 2);
  else if (n_rows <= 256 + 2) HISA_SW(1, 4);
  else if (n_rows <= 512 + 2) HISA_SW(1, 8);
  else if (n_rows <= 1024 + 2) HISA_SW(1, 16);
  else if (n_rows <= 16 * 1024 && (m - 2) * 16 <= kSelUnion) HISA_SW(16, 16);
#undef HISA_SW
  // many kept blocks: the workgroup-wide histogram select
  else if (n_rows <= 1024 * 16)
    hipLaunchKernelGGL((select_blocks_kernel<1024, 16, true>), grid, dim3(1024), 0, s, scores,
                       q_pos, nq, n_rows, B, m, block_idx);
  else
    hipLaunchKernelGGL((select_blocks_kernel<1024, 16, false>), grid, dim3(1024), 0, s, scores,
                       q_pos, nq, n_rows, B, m, block_idx);
  return hipGetLastError();
}

// ------------------------------------------------------- steps 2 and 3 fused
// For many queries over at most 64*16 + 2 blocks. A workgroup scores 16
// consecutive queries of one sequence against every causal candidate block
// into LDS, with the same exact three-term products (and summation order) as
// block_score_kernel, then each of its 8 waves selects the top blocks of two
// of the queries from LDS as select_blocks_wave_kernel does, so the score matrix
// never reaches HBM and the result equals the two kernels' bit for bit.
// Workgroups are dealt to the 8 XCDs in contiguous runs of (sequence, query
// tile), so an XCD's L2 serves few sequences' summary tables.
constexpr int kRouteQT = 16;

constexpr int kRouteWaves = 8;

template <int D, int IT>
__global__ __launch_bounds__(64 * kRouteWaves) void route_blocks_kernel(
    const uint16_t* __restrict__ qidx, int64_t qsb, int64_t qst, const int32_t* __restrict__ q_pos,
    int nq, const uint16_t* __restrict__ split, int n_rows, int B, float invB, int m,
    int32_t* __restrict__ block_idx, int batch, int ntq, unsigned grid_wg) {
  constexpr int KS = D / 32;
  constexpr int NC = 64 * IT;  // candidate positions (position p is block p + 1)
  constexpr int LS = NC + 4;   // LDS floats per query row
  __shared__ __align__(16) float sc[kRouteQT][LS];
  __shared__ uint32_t lkey[kRouteWaves][kSelSmall];
  __shared__ int lpos[kRouteWaves][kSelSmall];
  const unsigned per = grid_wg / 8;
  const unsigned id = (blockIdx.x % 8) * per + blockIdx.x / 8;
  if (id >= static_cast<unsigned>(batch) * ntq) return;
  const int b = static_cast<int>(id / ntq), q0 = static_cast<int>(id % ntq) * kRouteQT;
  const int w = threadIdx.x >> 6, l = lane_id(), g = l / 16, r16 = l % 16;
  const int qq = q0 + r16;
  const int qc = min(qq, nq - 1);
  const int bt = qq < nq ? min(max(q_pos[static_cast<int64_t>(b) * nq + qc], 0), n_rows * B - 1) / B
                         : 0;
  const int btmax = static_cast<int>(wave_max(static_cast<float>(bt)));
  const uint16_t* qrow = qidx + b * qsb + static_cast<int64_t>(qc) * qst + 8 * g;
  bf16x8 qf[KS];
#pragma unroll
  for (int x = 0; x < KS; ++x) qf[x] = as_bf16x8(*reinterpret_cast<const uint4*>(qrow + 32 * x));
  // row tile tau: blocks 1 + 16 tau .. 16 + 16 tau (positions 16 tau ..);
  // wave w takes tiles w, w + NW, ..., two per step with all their loads in
  // flight before the first product
  constexpr int NW = kRouteWaves;
  const int ntile = btmax > 1 ? (btmax - 1 + 15) / 16 : 0;
  for (int tau = w; tau < ntile; tau += 2 * NW) {
    uint4 sf[2][3 * KS];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int cc = min(1 + 16 * (tau + u * NW) + r16, n_rows - 1);
      const uint16_t* srow = split + (static_cast<int64_t>(b) * n_rows + cc) * 3 * D + 8 * g;
#pragma unroll
      for (int x = 0; x < 3 * KS; ++x)
        sf[u][x] = *reinterpret_cast<const uint4*>(srow + (x / KS) * D + 32 * (x % KS));
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int tu = tau + u * NW;
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int x = 0; x < 3 * KS; ++x) acc = mfma16(as_bf16x8(sf[u][x]), qf[x % KS], acc);
      // lane: blocks 1 + 16 tu + 4g + (0..3) of query column r16
      if (tu < ntile)
        *reinterpret_cast<float4*>(&sc[r16][16 * tu + 4 * g]) =
            make_float4(acc[0] * invB, acc[1] * invB, acc[2] * invB, acc[3] * invB);
    }
  }
  __syncthreads();
  for (int j = w; j < kRouteQT; j += NW) {
    const int q = q0 + j;
    if (q >= nq) break;
    const int64_t qi = static_cast<int64_t>(b) * nq + q;
    int32_t* out = block_idx + qi * m;
    const int bq = min(max(q_pos[qi], 0), n_rows * B - 1) / B;
    const int n = max(bq - 1, 0);
    const int K = m - (bq == 0 ? 1 : 2);  // free slots
    if (n <= K) {
      for (int i = l; i < m; i += 64) out[i] = i <= bq ? i : -1;
      continue;
    }
    uint32_t key[IT];
    uint32_t okm = 0;
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int p = 64 * i + l;
      key[i] = p < n ? order_key(sc[j][p]) : 0u;
      okm |= p < n ? (1u << i) : 0u;
    }
    wave_topk(key, okm, static_cast<uint32_t>(K), lkey[w], lpos[w],
              [&](uint32_t pos, int p) { out[1 + pos] = p + 1; });
    if (l == 0) {
      out[0] = 0;
      out[1 + K] = bq;
    }
  }
}

// The same for any number of blocks, streaming: per step the 4 waves score
// 64 consecutive candidate blocks for the 16 queries (one 16-block tile
// each, the next step's summary rows loaded while this one is scored), the
// scores meet in LDS (double buffered, one barrier per step), and wave w
// filters the step's scores of queries w, w+4, w+8, w+12 against each
// query's threshold key, appending the survivors to the query's LDS buffer
// in position order. A buffer about to overflow is cut back to its best K
// (wave_select, ties to the lowest position since the buffer is in position
// order), whose K-th key becomes the threshold: a later block equal to it
// has a higher position and could not displace it. A last select over the
// buffer gives the kept blocks. K = m - 2 <= kStreamK.
// buffer entries per query: CAP >= K + 128 (a cut leaves K, at most 64 come
// per filtering round, a cut follows when more than CAP - 64 are held)
template <int D, int NW, int QS, int TW, int CAP>
__global__ __launch_bounds__(64 * NW) void route_blocks_stream_kernel(
    const uint16_t* __restrict__ qidx, int64_t qsb, int64_t qst, const int32_t* __restrict__ q_pos,
    int nq, const uint16_t* __restrict__ split, int n_rows, int B, float invB, int m,
    int32_t* __restrict__ block_idx, int batch, int ntq, unsigned grid_wg) {
  constexpr int KS = D / 32;
  constexpr int NQB = QS / 16;          // 16-query column blocks of the products
  constexpr int SB = 16 * NW * TW;      // candidate blocks per step (TW tiles per wave)
  constexpr int QW = QS / NW;           // queries filtered per wave
  __shared__ __align__(16) float stg[2][QS][SB];
  __shared__ uint32_t bkey[QS][CAP];
  __shared__ uint16_t bpos[QS][CAP];  // positions < 65536 (n_rows <= 65537)
  const unsigned per = grid_wg / 8;
  const unsigned id = (blockIdx.x % 8) * per + blockIdx.x / 8;
  if (id >= static_cast<unsigned>(batch) * ntq) return;
  const int b = static_cast<int>(id / ntq), q0 = static_cast<int>(id % ntq) * QS;
  const int w = threadIdx.x >> 6, l = lane_id(), g = l / 16, r16 = l % 16;
  bf16x8 qf[NQB][KS];
  int bt[NQB];
  int btm = 0;
#pragma unroll
  for (int cb = 0; cb < NQB; ++cb) {
    const int qq = q0 + 16 * cb + r16;
    const int qc = min(qq, nq - 1);
    bt[cb] = qq < nq
                 ? min(max(q_pos[static_cast<int64_t>(b) * nq + qc], 0), n_rows * B - 1) / B
                 : 0;
    btm = max(btm, bt[cb]);
    const uint16_t* qrow = qidx + b * qsb + static_cast<int64_t>(qc) * qst + 8 * g;
#pragma unroll
    for (int x = 0; x < KS; ++x)
      qf[cb][x] = as_bf16x8(*reinterpret_cast<const uint4*>(qrow + 32 * x));
  }
  const int btmax = static_cast<int>(wave_max(static_cast<float>(btm)));
  // this wave's queries: candidates, free slots, threshold, buffer fill
  int nc[QW], kq[QW], cnt[QW];
  uint32_t th[QW];
#pragma unroll
  for (int u = 0; u < QW; ++u) {
    const int j = w + NW * u;
    int bq = 0;
#pragma unroll
    for (int cb = 0; cb < NQB; ++cb) {
      const int v = __shfl(bt[cb], j % 16, 64);
      bq = j / 16 == cb ? v : bq;
    }
    nc[u] = q0 + j < nq ? max(bq - 1, 0) : 0;
    kq[u] = m - (bq == 0 ? 1 : 2);
    th[u] = 0u;
    cnt[u] = 0;
  }
  const int nsteps = btmax > 1 ? (btmax - 1 + SB - 1) / SB : 0;
  // wave w scores tiles w, w + NW, ... (TW of them) of each step
  auto load = [&](int step, uint4 (&sf)[TW][3 * KS]) {
#pragma unroll
    for (int v = 0; v < TW; ++v) {
      const int cc = min(1 + SB * step + 16 * (w + NW * v) + r16, n_rows - 1);
      const uint16_t* srow = split + (static_cast<int64_t>(b) * n_rows + cc) * 3 * D + 8 * g;
#pragma unroll
      for (int x = 0; x < 3 * KS; ++x)
        sf[v][x] = *reinterpret_cast<const uint4*>(srow + (x / KS) * D + 32 * (x % KS));
    }
  };
  uint4 sf[TW][3 * KS];
  if (nsteps > 0) load(0, sf);
  for (int step = 0; step < nsteps; ++step) {
    f32x4 acc[TW][NQB];
#pragma unroll
    for (int v = 0; v < TW; ++v)
#pragma unroll
      for (int cb = 0; cb < NQB; ++cb) {
        acc[v][cb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int x = 0; x < 3 * KS; ++x)
          acc[v][cb] = mfma16(as_bf16x8(sf[v][x]), qf[cb][x % KS], acc[v][cb]);
      }
    if (step + 1 < nsteps) load(step + 1, sf);
    float* sg = &stg[step & 1][0][0];
#pragma unroll
    for (int v = 0; v < TW; ++v)
#pragma unroll
      for (int cb = 0; cb < NQB; ++cb)
        *reinterpret_cast<float4*>(sg + (16 * cb + r16) * SB + 16 * (w + NW * v) + 4 * g) =
            make_float4(acc[v][cb][0] * invB, acc[v][cb][1] * invB, acc[v][cb][2] * invB,
                        acc[v][cb][3] * invB);
    __syncthreads();
#pragma unroll
    for (int u = 0; u < QW; ++u) {
      const int j = w + NW * u;
      // key > th as a float compare: the key order is the float order (with
      // -0 == +0), and th = 0 (no cut yet) passes every score, as NaN does
      const float thf = th[u] == 0u ? __uint_as_float(0x7fc00000u) : key_value(th[u]);
#pragma unroll
      for (int h = 0; h < SB / 64; ++h) {
        const int p = SB * step + 64 * h + l;
        const float x = sg[j * SB + 64 * h + l];
        const bool pass = p < nc[u] && !(x <= thf);
        const uint64_t pm = __ballot(pass);
        if (pm == 0ull) continue;
        if (pass) {
          const int e = cnt[u] + static_cast<int>(lanes_below(pm));
          bkey[j][e] = order_key(x);
          bpos[j][e] = p;
        }
        cnt[u] += static_cast<int>(__popcll(pm));
        if (cnt[u] > CAP - 64) {
          // cut the buffer back to its best kq (in position order)
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
          uint32_t k2[CAP / 64];
          int p2[CAP / 64];
          uint32_t ok2 = 0;
#pragma unroll
          for (int i = 0; i < CAP / 64; ++i) {
            const int e = 64 * i + l;
            k2[i] = e < cnt[u] ? bkey[j][e] : 0u;
            p2[i] = e < cnt[u] ? bpos[j][e] : 0;
            ok2 |= e < cnt[u] ? (1u << i) : 0u;
          }
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
          const WaveSel sel = wave_select(k2, ok2, static_cast<uint32_t>(kq[u]));
          wave_compact(k2, ok2, sel, [&](int i, uint32_t pos) {
            bkey[j][pos] = k2[i];
            bpos[j][pos] = p2[i];
          });
          th[u] = sel.T;
          cnt[u] = kq[u];
        }
      }
    }
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
#pragma unroll
  for (int u = 0; u < QW; ++u) {
    const int j = w + NW * u;
    const int q = q0 + j;
    if (q >= nq) break;
    const int64_t qi = static_cast<int64_t>(b) * nq + q;
    int32_t* out = block_idx + qi * m;
    const int bq = nc[u] + 1;  // blocks 1 .. bq-1 are the candidates (bq = t / B when t >= B)
    if (nc[u] <= kq[u]) {
      const int bqq = min(max(q_pos[qi], 0), n_rows * B - 1) / B;
      for (int i = l; i < m; i += 64) out[i] = i <= bqq ? i : -1;
      continue;
    }
    uint32_t k2[CAP / 64];
    uint32_t ok2 = 0;
#pragma unroll
    for (int i = 0; i < CAP / 64; ++i) {
      const int e = 64 * i + l;
      k2[i] = e < cnt[u] ? bkey[j][e] : 0u;
      ok2 |= e < cnt[u] ? (1u << i) : 0u;
    }
    const WaveSel sel = wave_select(k2, ok2, static_cast<uint32_t>(kq[u]));
    wave_compact(k2, ok2, sel, [&](int i, uint32_t pos) { out[1 + pos] = bpos[j][64 * i + l] + 1; });
    if (l == 0) {
      out[0] = 0;
      out[1 + kq[u]] = bq;
    }
  }
}

// ----------------------------------------- steps 2 and 3 for few queries
// Few queries over many blocks leave most of the chip idle when each query
// is scored and selected by one workgroup. Here each query's candidate
// positions are cut into parts of kPart: a workgroup of four waves scores
// one part (the exact three-term products of block_score_kernel in its
// summation order, so the scores are the same bits) into LDS, and its first
// wave keeps the part's best K = m - 2 (wave_topk: ties to the lowest
// position) in the workspace as (order key, position) pairs, in position
// order. One wave per query then takes the best K of the parts' survivors:
// every overall winner is a winner of its part under the same order, and
// the survivors, part after part, are in position order, so ties again go to
// the lowest position. It adds the first and the local block around them.
constexpr int kPart = 256;
constexpr int kSplitMaxK = 64;        // free slots: wave_topk's short path
constexpr int kSplitMaxUnion = 2048;  // survivors per query the merge holds

constexpr int kPartWaves = kPart / 32;  // each wave scores two 16-row tiles, one load round

template <int D>
__global__ __launch_bounds__(64 * kPartWaves) void route_part_kernel(
    const uint16_t* __restrict__ qidx, int64_t qsb, int64_t qst, const int32_t* __restrict__ q_pos,
    int nq, const uint16_t* __restrict__ split, int n_rows, int B, float invB, int m,
    uint2* __restrict__ parts, int nparts) {
  constexpr int KS = D / 32;
  __shared__ __align__(16) float sc[kPart];
  __shared__ uint32_t lkey[kSelSmall];
  __shared__ int lpos[kSelSmall];
  const int part = blockIdx.x;
  const int64_t qi = blockIdx.y;
  const int b = static_cast<int>(qi / nq), q = static_cast<int>(qi % nq);
  const int bt = min(max(q_pos[qi], 0), n_rows * B - 1) / B;
  const int n = max(bt - 1, 0);
  const int K = m - 2;
  const int p0 = part * kPart;
  if (n <= K || p0 >= n) return;  // all blocks kept, or no candidate here: the merge
  const int w = threadIdx.x >> 6, l = lane_id(), g = l / 16, r16 = l % 16;
  const int cnt = min(kPart, n - p0);
  if (32 * w < cnt) {
    // every column of the products is this query (one column is stored)
    const uint16_t* qrow = qidx + b * qsb + static_cast<int64_t>(q) * qst + 8 * g;
    bf16x8 qf[KS];
#pragma unroll
    for (int x = 0; x < KS; ++x) qf[x] = as_bf16x8(*reinterpret_cast<const uint4*>(qrow + 32 * x));
    // wave w: local positions 32w + 16u + (0..15), u = 0, 1 (position p is
    // block p + 1), all loads of both tiles in flight before the products
    uint4 sf[2][3 * KS];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int cc = min(1 + p0 + 32 * w + 16 * u + r16, n_rows - 1);
      const uint16_t* srow = split + (static_cast<int64_t>(b) * n_rows + cc) * 3 * D + 8 * g;
#pragma unroll
      for (int x = 0; x < 3 * KS; ++x)
        sf[u][x] = *reinterpret_cast<const uint4*>(srow + (x / KS) * D + 32 * (x % KS));
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int x = 0; x < 3 * KS; ++x) acc = mfma16(as_bf16x8(sf[u][x]), qf[x % KS], acc);
      // lane (g, column r16): local positions 32w + 16u + 4g + (0..3)
      if (r16 == 0)
        *reinterpret_cast<float4*>(&sc[32 * w + 16 * u + 4 * g]) =
            make_float4(acc[0] * invB, acc[1] * invB, acc[2] * invB, acc[3] * invB);
    }
  }
  __syncthreads();
  if (w == 0) {
    uint32_t key[kPart / 64];
    uint32_t okm = 0;
#pragma unroll
    for (int i = 0; i < kPart / 64; ++i) {
      const int p = 64 * i + l;
      key[i] = p < cnt ? order_key(sc[p]) : 0u;
      okm |= p < cnt ? (1u << i) : 0u;
    }
    uint2* dst = parts + (qi * nparts + part) * K;
    wave_topk(key, okm, static_cast<uint32_t>(min(K, cnt)), lkey, lpos,
              [&](uint32_t rank, int p) {
                dst[rank] = make_uint2(order_key(sc[p]), static_cast<uint32_t>(p0 + p));
              });
  }
}

// Entry e = u*K + j is survivor j of part u; part u keeps min(K, its
// candidates). With W waves, wave v reduces parts v*PW .. v*PW + PW - 1 to
// their best K (in position order, into LDS), and wave 0 takes the best K of
// those W*K; IT and IT2 items per lane hold the two stages.
template <int W, int IT, int IT2>
__global__ __launch_bounds__(64 * W) void route_merge_kernel(const int32_t* __restrict__ q_pos,
                                                             int n_rows, int B, int m,
                                                             const uint2* __restrict__ parts,
                                                             int nparts, int PW,
                                                             int32_t* __restrict__ block_idx) {
  __shared__ uint32_t lkey[W][kSelSmall];
  __shared__ int lpos[W][kSelSmall];
  __shared__ uint32_t ukey[W > 1 ? W * kSplitMaxK : 1];
  __shared__ int upos[W > 1 ? W * kSplitMaxK : 1];
  __shared__ int ucnt[W];
  const int64_t qi = blockIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), l = lane_id();
  const int bt = min(max(q_pos[qi], 0), n_rows * B - 1) / B;
  const int n = max(bt - 1, 0);
  const int K = m - (bt == 0 ? 1 : 2);
  int32_t* out = block_idx + qi * m;
  if (n <= K) {
    for (int i = threadIdx.x; i < m; i += 64 * W) out[i] = i <= bt ? i : -1;
    return;
  }
  const int np = (n + kPart - 1) / kPart;
  const uint2* src = parts + qi * nparts * K;
  // this wave's entries: parts w*PW .. (their survivors, in position order)
  const int u0 = w * PW;
  const int nu = max(0, min(PW, np - u0));
  uint32_t key[IT];
  uint32_t okm = 0;
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const int e = 64 * i + l;  // entry of this wave's range
    const int u = e / K, j = e - u * K;
    const bool ok = u < nu && j < min(K, n - (u0 + u) * kPart);
    const uint32_t k = src[ok ? u0 * K + e : 0].x;  // entry 0 exists: the query has candidates
    key[i] = ok ? k : 0u;
    okm |= ok ? (1u << i) : 0u;
  }
  if constexpr (W == 1) {
    wave_topk(key, okm, static_cast<uint32_t>(K), lkey[0], lpos[0],
              [&](uint32_t rank, int e) { out[1 + rank] = static_cast<int32_t>(src[e].y) + 1; });
  } else {
    // this wave's best min(K, its entries) into LDS, in position order
    uint32_t have = 0;
#pragma unroll
    for (int i = 0; i < IT; ++i) have += static_cast<uint32_t>(__popcll(__ballot((okm >> i) & 1u)));
    const uint32_t kv = min(static_cast<uint32_t>(K), have);
    if (kv > 0)
      wave_topk(key, okm, kv, lkey[w], lpos[w], [&](uint32_t rank, int e) {
        ukey[w * kSplitMaxK + rank] = src[u0 * K + e].x;
        upos[w * kSplitMaxK + rank] = static_cast<int>(src[u0 * K + e].y);
      });
    if (l == 0) ucnt[w] = static_cast<int>(kv);
    __syncthreads();
    if (w == 0) {
      // entry f = v*kSplitMaxK + r: survivor r of wave v (position order)
      uint32_t k2[IT2];
      uint32_t ok2 = 0;
#pragma unroll
      for (int i = 0; i < IT2; ++i) {
        const int f = 64 * i + l;
        const int v = f / kSplitMaxK, r = f % kSplitMaxK;
        const bool ok = v < W && r < ucnt[min(v, W - 1)];
        k2[i] = ok ? ukey[min(f, W * kSplitMaxK - 1)] : 0u;
        ok2 |= ok ? (1u << i) : 0u;
      }
      wave_topk(k2, ok2, static_cast<uint32_t>(K), lkey[0], lpos[0],
                [&](uint32_t rank, int f) { out[1 + rank] = upos[f] + 1; });
    }
  }
  if (threadIdx.x == 0) {
    out[0] = 0;
    out[1 + K] = bt;
  }
}

// Parts per query for the split routing, or 0 when it does not apply.
static int route_split_parts(int64_t nqueries, int n_rows, int m) {
  if (nqueries >= 1024 || m < 3 || m - 2 > kSplitMaxK || n_rows > kRouteStreamMaxRows) return 0;
  const int nmax = max(n_rows - 2, 0);  // candidates of the last block's queries
  const int nparts = max(1, (nmax + kPart - 1) / kPart);
  if (static_cast<int64_t>(nparts) * (m - 2) > kSplitMaxUnion) return 0;
  return nparts;
}

size_t route_split_workspace(int batch, int nq, int n_rows, int m) {
  const int64_t nqt = static_cast<int64_t>(batch) * nq;
  const int nparts = route_split_parts(nqt, n_rows, m);
  if (nparts == 0) return 0;
  return align256(static_cast<size_t>(nqt) * nparts * (m - 2) * sizeof(uint2));
}

static hipError_t launch_route_split(const uint16_t* qidx, Str3 qs, const int32_t* q_pos,
                                     int batch, int nq, const uint16_t* split, int n_rows, int d,
                                     int B, int m, int32_t* block_idx, void* ws, hipStream_t s) {
  const int64_t nqt = static_cast<int64_t>(batch) * nq;
  const int nparts = route_split_parts(nqt, n_rows, m);
  const float invB = 1.0f / static_cast<float>(B);
  uint2* parts = static_cast<uint2*>(ws);
  const dim3 g1(static_cast<unsigned>(nparts), static_cast<unsigned>(nqt));
  if (d == 64)
    hipLaunchKernelGGL(route_part_kernel<64>, g1, dim3(64 * kPartWaves), 0, s, qidx, qs.b, qs.t,
                       q_pos, nq, split, n_rows, B, invB, m, parts, nparts);
  else
    hipLaunchKernelGGL(route_part_kernel<128>, g1, dim3(64 * kPartWaves), 0, s, qidx, qs.b,
                       qs.t, q_pos, nq, split, n_rows, B, invB, m, parts, nparts);
  // merge: one wave while the survivors fit four items per lane, else four
  // waves, each over a quarter of the parts (ceil(nparts / 4) * K <= 560
  // entries since nparts * K <= 2048 and K <= 64), then wave 0 over their
  // best K each
  const int K = m - 2;
  const dim3 g2(static_cast<unsigned>(nqt));
  if (nparts * K <= 256) {
    hipLaunchKernelGGL((route_merge_kernel<1, 4, 1>), g2, dim3(64), 0, s, q_pos, n_rows, B, m,
                       parts, nparts, nparts, block_idx);
  } else {
    const int pw = (nparts + 3) / 4;  // parts per wave
    hipLaunchKernelGGL((route_merge_kernel<4, 9, 4>), g2, dim3(256), 0, s, q_pos, n_rows, B, m,
                       parts, nparts, pw, block_idx);
  }
  return hipGetLastError();
}

hipError_t launch_route_blocks(const uint16_t* qidx, Str3 qs, const int32_t* q_pos, int batch,
                               int nq, const uint16_t* split, int n_rows, int d, int B, int m,
                               int32_t* block_idx, void* ws, hipStream_t s) {
  if (ws != nullptr && route_split_workspace(batch, nq, n_rows, m) > 0)
    return launch_route_split(qidx, qs, q_pos, batch, nq, split, n_rows, d, B, m, block_idx, ws,
                              s);
  const int ntq = (nq + kRouteQT - 1) / kRouteQT;
  const unsigned grid_wg =
      static_cast<unsigned>((static_cast<int64_t>(batch) * ntq + 7) / 8 * 8);
  const float invB = 1.0f / static_cast<float>(B);
  // streamed selection whenever m allows it: faster than holding all scores
  // on chip even at 1024 blocks (64K two-level prefill routing 2.72 -> 2.39
  // ms). With many blocks (more than 3072) and up to 64 free slots, 32
  // queries per workgroup with 128-entry buffers: each summary row load feeds
  // twice the products at the same 40 KB of LDS (512K routing 89 -> 66 ms,
  // 256K 24.3 -> 22.1; at 2048 blocks 7.0 -> 7.6, so fewer blocks keep 16
  // queries and 256 entries, as does m above 66).
  if (m <= kRouteStreamMaxM && n_rows <= kRouteStreamMaxRows) {
    auto go = [&](auto nw, auto qsz, auto cap) {
      constexpr int NW = decltype(nw)::value, QS = decltype(qsz)::value;
      constexpr int CAP = decltype(cap)::value;
      const int ntq_s = (nq + QS - 1) / QS;
      const unsigned grid_s =
          static_cast<unsigned>((static_cast<int64_t>(batch) * ntq_s + 7) / 8 * 8);
      if (d == 64)
        hipLaunchKernelGGL((route_blocks_stream_kernel<64, NW, QS, 1, CAP>), dim3(grid_s),
                           dim3(64 * NW), 0, s, qidx, qs.b, qs.t, q_pos, nq, split, n_rows, B,
                           invB, m, block_idx, batch, ntq_s, grid_s);
      else
        hipLaunchKernelGGL((route_blocks_stream_kernel<128, NW, QS, 1, CAP>), dim3(grid_s),
                           dim3(64 * NW), 0, s, qidx, qs.b, qs.t, q_pos, nq, split, n_rows, B,
                           invB, m, block_idx, batch, ntq_s, grid_s);
    };
    if (m - 2 <= 64 && n_rows > 3072)
      go(std::integral_constant<int, 4>{}, std::integral_constant<int, 32>{},
         std::integral_constant<int, 128>{});
    else
      go(std::integral_constant<int, 4>{}, std::integral_constant<int, 16>{},
         std::integral_constant<int, 256>{});
    return hipGetLastError();
  }
#define HISA_RB(D_, IT_)                                                                        \
  hipLaunchKernelGGL((route_blocks_kernel<D_, IT_>), dim3(grid_wg), dim3(64 * kRouteWaves), 0, s, \
                     qidx, qs.b,                                                                \
                     qs.t, q_pos, nq, split, n_rows, B, invB, m, block_idx, batch, ntq, grid_wg)
#define HISA_RB_D(IT_)              \
  do {                              \
    if (d == 64) HISA_RB(64, IT_);  \
    else HISA_RB(128, IT_);         \
  } while (0)
  if (n_rows <= 64 + 2) HISA_RB_D(1);
  else if (n_rows <= 128 + 2) HISA_RB_D(2);
  else if (n_rows <= 256 + 2) HISA_RB_D(4);
  else if (n_rows <= 512 + 2) HISA_RB_D(8);
  else HISA_RB_D(16);
#undef HISA_RB_D
#undef HISA_RB
  return hipGetLastError();
}

}  // namespace hisa
