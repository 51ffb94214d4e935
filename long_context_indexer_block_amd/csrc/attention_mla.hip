// Sparse attention for multi-head latent attention rows: 64 query heads read
// one latent row per token of width 576, whose first 512 columns are also the
// value row. This is the shape of the 64K prefill workload and dominates its
// time (HISA explainer 1.1: attention over the selected tokens only; HISA
// news article: the downstream attention is unchanged).
//
// One workgroup (4 waves, one per SIMD) per query. Per tile of 64 selected
// tokens:
//   * the 64 latent rows are gathered from HBM straight into LDS with 16-byte
//     direct loads (global_load_lds), one tile ahead of the compute, into one
//     of two statically distinct LDS tiles; the 16-byte chunks of each row
//     are XOR-swizzled so every matrix-core fragment read is free of bank
//     conflicts (the lane -> chunk assignment of the loads realises the
//     swizzle while keeping each 128-byte line read by 8 adjacent lanes);
//   * S^T = K Q^T on 32x32x16 bf16 MFMA: wave (hh, tt) owns heads 32hh..+32
//     and tokens 32tt..+32 with its Q rows resident in registers for the
//     whole query; in the S^T layout each lane holds one head column, so the
//     softmax row statistics need one cross-lane step;
//   * online softmax in base 2 (fp32), P written to LDS as bf16;
//   * O^T = V^T P^T: wave (hh, dd) owns heads 32hh..+32 and value columns
//     256dd..+256; V^T fragments come straight from the row-major latent
//     tile through ds_read_tr16_b64 (each 16-lane group turns a 4-token x
//     16-column block into 16 columns of 4 tokens), so V is never copied.
//     O stays in registers (128 fp32 per lane) until the end.
// Barriers are plain s_barrier after an LDS-counter wait, so the in-flight
// tile load is never drained early. Workgroups are mapped so each XCD walks
// a contiguous range of queries: neighbouring queries share their forced
// blocks and sweep the same token range together, which raises L2 reuse.
#include "common.hpp"
#include "internal.h"

namespace hisa {
namespace mla {

constexpr int H = 64, DK = 576, DV = 512, NT = 64;
constexpr int RCH = DK / 8;     // 16-byte chunks per latent row (72)
constexpr int PITCH = RCH + 1;  // LDS row pitch in chunks: odd, so 16 rows at one chunk
                                // (292 words apart, 36 mod 64) hit distinct banks
constexpr int TSL = NT * PITCH; // chunk slots per tile (4672 = 73 load instructions)
constexpr int KS = DK / 16;     // k steps of S (36)
constexpr int PP = 9;           // P row pitch in chunks (8 + 1)

typedef __attribute__((address_space(3))) void* lds_ptr;
typedef __attribute__((address_space(1))) void* glb_ptr;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short v4s;

__device__ __forceinline__ uint2 tr16(const unsigned char* lds_byte) {
  const v4s v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4s*)(lds_byte));
  return __builtin_bit_cast(uint2, v);
}
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// LDS-only barrier: wait for this wave's LDS operations, then s_barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
}

__shared__ uint4 g_tile_a[TSL];
__shared__ uint4 g_tile_b[TSL];
__shared__ uint4 g_p[H * PP];       // P as [head][8 chunks of 8 tokens] + 1 pad chunk
__shared__ float g_mx[2][H];
__shared__ float g_lsum[2][H];

// Gather the 64 latent rows of one tile into `dst` (row r, chunk c at slot
// r*PITCH + c). The 73 direct-to-LDS instructions of a tile each fill 64
// consecutive slots (wave 0 issues 19, the others 18); lane l of
// instruction i takes slot s = 64i + l, i.e. row s / PITCH, chunk s % PITCH
// (the pad chunk re-reads chunk 71). Adjacent lanes read adjacent 16-byte
// chunks of a row, so the loads are coalesced.
__device__ __forceinline__ void dma_tile(uint4* dst, const uint16_t* kvb, int64_t kst, int ids,
                                         int w, int l) {
  const int i0 = w == 0 ? 0 : 19 + 18 * (w - 1);
  const int cnt = w == 0 ? 19 : 18;
#pragma unroll
  for (int j = 0; j < 19; ++j) {
    if (j < cnt) {
      const int s = 64 * (i0 + j) + l;
      const int r = s / PITCH, c = s - r * PITCH;
      const int id = __shfl(ids, r, kWave);
      const uint16_t* src = kvb + static_cast<int64_t>(id < 0 ? 0 : id) * kst + 8 * min(c, RCH - 1);
      __builtin_amdgcn_global_load_lds((glb_ptr)(src), (lds_ptr)(dst + 64 * (i0 + j)), 16, 0, 0);
    }
  }
}

struct State {
  bf16x8 qf[KS];
  f32x16 o[8];
  float m_run, l_run;
};

// One tile: S^T, softmax, P, O^T update. `cur` holds the tile; the next
// tile's loads into `nxt` are issued first, always (past the last tile every
// id is -1 and the loads fetch row 0 again, which hits in cache), so the
// code is straight-line and the compiler's load-counter waits stay exact.
__device__ __forceinline__ void tile_step(const uint4* cur, uint4* nxt, State& st,
                                          int& ids_cur, int& ids_next, const int32_t* tix, int topk,
                                          int L, int tile, const uint16_t* kvb, int64_t kst,
                                          float scale_log2, int w, int l) {
  // Opaque copy of the lane id: address arithmetic derived from it is redone
  // per tile instead of being hoisted into long-lived registers.
  asm volatile("" : "+v"(l));
  const int hh = w >> 1, tt = w & 1, l32 = l & 31, lh = l >> 5;
  const int head = 32 * hh + l32;
  // tile `tile` (in cur) and the ids of tile+1 are complete for this wave
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  const uint64_t vmask = __ballot(ids_cur >= 0);
  // ids of tile+2 are loaded before the tile+1 gather: load counters retire
  // in order, so waiting for the ids later never drains the gather
  const int idx = (tile + 2) * NT + l;
  int jraw = tix[min(idx, topk - 1)];
  dma_tile(nxt, kvb, kst, ids_next, w, l);
  ids_cur = ids_next;
  ids_next = (idx < topk && jraw >= 0 && jraw < L) ? jraw : -1;

  // ---- S^T[tokens 32tt + (0..31)][heads 32hh + (0..31)] = K Q^T
  f32x16 sacc;
#pragma unroll
  for (int e = 0; e < 16; ++e) sacc[e] = 0.0f;
  {
    const uint4* ka = cur + (32 * tt + l32) * PITCH + lh;
#pragma unroll
    for (int s = 0; s < KS; ++s) sacc = mfma32(as_bf16x8(ka[2 * s]), st.qf[s], sacc);
  }
  float sv[16];
  float mloc = -INFINITY;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int tk = 32 * tt + 8 * (e >> 2) + 4 * lh + (e & 3);
    sv[e] = ((vmask >> tk) & 1ull) ? sacc[e] * scale_log2 : -INFINITY;
    mloc = fmaxf(mloc, sv[e]);
  }
  mloc = fmaxf(mloc, __shfl_xor(mloc, 32, kWave));
  if (lh == 0) g_mx[tt][head] = mloc;
  lds_barrier();
  // Lazy rescaling: the reference maximum moves only when the tile maximum
  // exceeds it by more than 8 (a factor 256 in p), so most tiles leave O
  // untouched. Every lane holding a head takes the same decision.
  const float mtile = fmaxf(mloc, g_mx[tt ^ 1][head]);
  const bool move = mtile > st.m_run + 8.0f;
  const float mref = move ? mtile : st.m_run;
  const float alpha = move ? exp2f(st.m_run - mtile) : 1.0f;
  float psum = 0.0f;
  uint32_t pk[8];
#pragma unroll
  for (int e = 0; e < 16; e += 2) {
    const uint16_t a = f32_to_bf16(exp2f(sv[e] - mref));
    const uint16_t c = f32_to_bf16(exp2f(sv[e + 1] - mref));
    psum += bf16_to_f32(a) + bf16_to_f32(c);
    pk[e >> 1] = static_cast<uint32_t>(a) | (static_cast<uint32_t>(c) << 16);
  }
  st.m_run = mref;
  st.l_run = st.l_run * alpha + psum;
  // P[head][token 32tt + 8q + 4lh + (0..3)]: chunk 4tt + q, half lh
  {
    uint2* prow = reinterpret_cast<uint2*>(g_p + head * PP + 4 * tt) + lh;
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) prow[2 * qq] = make_uint2(pk[2 * qq], pk[2 * qq + 1]);
  }
  if (__ballot(move) != 0ull) {
#pragma unroll
    for (int d = 0; d < 8; ++d)
#pragma unroll
      for (int e = 0; e < 16; ++e) st.o[d][e] *= alpha;
  }
  lds_barrier();

  // ---- O^T[dv 256tt + 32dt + (0..31)][heads] += V^T P^T over the tile's 64 tokens
  {
    const int G = l >> 4, sl = l & 15;
    const int trow = 8 * (G >> 1) + (sl >> 2);
    const int dcol = 16 * (G & 1) + 4 * (sl & 3);
    // token row 16s + trow + 4h, value column 256tt + 32dt + dcol: one base
    // address per lane, everything else a compile-time offset
    const unsigned char* vb = reinterpret_cast<const unsigned char*>(cur) +
                              16 * (trow * PITCH + 32 * tt + (dcol >> 3)) + 2 * (dcol & 7);
    const uint4* pa = g_p + head * PP + lh;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const bf16x8 pb = as_bf16x8(pa[2 * s]);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const int off = 16 * ((16 * s) * PITCH + 4 * dt);
        const uint2 lo = tr16(vb + off);
        const uint2 hi = tr16(vb + off + 16 * 4 * PITCH);
        st.o[dt] = mfma32(as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y)), pb, st.o[dt]);
      }
    }
  }
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_attn_kernel(const uint16_t* __restrict__ q, Str3 qs, const uint16_t* __restrict__ kv,
                     Str3 ks, int nq, int L, int Hkv, const int32_t* __restrict__ token_idx,
                     int topk, float scale_log2, uint16_t* __restrict__ out, Str3 os,
                     float* __restrict__ lse) {
  const int per = (nq + 7) / 8;
  const int qi = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (qi >= nq) return;
  const int b = blockIdx.y / Hkv, g = blockIdx.y % Hkv;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
  const int hh = w >> 1, tt = w & 1, l32 = l & 31, lh = l >> 5;
  const int head = 32 * hh + l32;
  const int64_t qrow = static_cast<int64_t>(b) * nq + qi;
  const int32_t* tix = token_idx + qrow * topk;
  const int ntiles = (topk + NT - 1) / NT;
  const uint16_t* kvb = kv + b * ks.b + g * ks.h;

  State st;
  {
    const uint16_t* qp = q + b * qs.b + qi * qs.t + (g * H + head) * qs.h + 8 * lh;
#pragma unroll
    for (int s = 0; s < KS; ++s) st.qf[s] = as_bf16x8(*reinterpret_cast<const uint4*>(qp + 16 * s));
  }
#pragma unroll
  for (int d = 0; d < 8; ++d)
#pragma unroll
    for (int e = 0; e < 16; ++e) st.o[d][e] = 0.0f;
  st.m_run = -INFINITY;
  st.l_run = 0.0f;
  auto read_id = [&](int idx) -> int {
    const int j = tix[min(idx, topk - 1)];
    return (idx < topk && j >= 0 && j < L) ? j : -1;
  };
  int ids_cur = read_id(l);
  dma_tile(g_tile_a, kvb, ks.t, ids_cur, w, l);
  int ids_next = read_id(NT + l);

  // an odd tile count gets one extra, fully masked tile
  for (int i = 0; i < ntiles; i += 2) {
    tile_step(g_tile_a, g_tile_b, st, ids_cur, ids_next, tix, topk, L, i, kvb, ks.t, scale_log2,
              w, l);
    tile_step(g_tile_b, g_tile_a, st, ids_cur, ids_next, tix, topk, L, i + 1, kvb, ks.t,
              scale_log2, w, l);
  }
  // drain the last (dummy) gather before the tile memory is reused below
  __builtin_amdgcn_s_waitcnt(0x0070);
  // ---- normalise: row sum over the lane pair and both token halves
  const float lw = st.l_run + __shfl_xor(st.l_run, 32, kWave);
  if (lh == 0) g_lsum[tt][head] = lw;
  __syncthreads();
  const float ltot = g_lsum[0][head] + g_lsum[1][head];
  const float inv = ltot > 0.0f ? 1.0f / ltot : 0.0f;
  // stage O as [head][512] bf16 in the first tile buffer, then store rows
  uint16_t* ost = reinterpret_cast<uint16_t*>(g_tile_a);
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d = 256 * tt + 32 * dt + 8 * q4 + 4 * lh;
      const uint32_t a = pack_bf16x2(st.o[dt][4 * q4 + 0] * inv, st.o[dt][4 * q4 + 1] * inv);
      const uint32_t c = pack_bf16x2(st.o[dt][4 * q4 + 2] * inv, st.o[dt][4 * q4 + 3] * inv);
      *reinterpret_cast<uint2*>(ost + head * DV + d) = make_uint2(a, c);
    }
  if (lse != nullptr && lh == 0 && tt == 0)
    lse[qrow * (static_cast<int64_t>(H) * Hkv) + g * H + head] =
        ltot > 0.0f ? (st.m_run + log2f(ltot)) * 0.69314718055994530942f : -INFINITY;
  __syncthreads();
  uint16_t* ob = out + b * os.b + qi * os.t + g * H * os.h;
#pragma unroll
  for (int j = 0; j < (H * DV / 8) / 256; ++j) {
    const int u = tid + 256 * j;
    const int hr = u / (DV / 8), c = u % (DV / 8);
    *reinterpret_cast<uint4*>(ob + hr * os.h + 8 * c) =
        *reinterpret_cast<const uint4*>(ost + hr * DV + 8 * c);
  }
}

}  // namespace mla

hipError_t launch_mla_attn(const uint16_t* q, Str3 qs, const uint16_t* kv, Str3 ks, int batch,
                           int nq, int L, int Hkv, const int32_t* token_idx, int topk, float scale,
                           uint16_t* out, Str3 os, float* lse, hipStream_t s) {
  const int per = (nq + 7) / 8;
  hipLaunchKernelGGL(mla::mla_attn_kernel, dim3(8 * per, batch * Hkv), dim3(256), 0, s, q, qs,
                     kv, ks, nq, L, Hkv, token_idx, topk, scale * 1.44269504088896340736f, out,
                     os, lse);
  return hipGetLastError();
}

}  // namespace hisa
