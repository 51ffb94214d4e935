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
constexpr int TCH = NT * RCH;   // chunk slots per tile (4608)
constexpr int KS = DK / 16;     // k steps of S (36)
constexpr int PP = 8;           // P row pitch in chunks

typedef __attribute__((address_space(3))) void* lds_ptr;
typedef __attribute__((address_space(1))) void* glb_ptr;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short v4s;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint2 tr16(const unsigned char* lds_byte) {
  const v4s v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4s*)(lds_byte));
  return __builtin_bit_cast(uint2, v);
}
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
// LDS-only barrier: wait for this wave's LDS operations, then s_barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
}

__shared__ uint4 g_tile_a[TCH];
__shared__ uint4 g_tile_b[TCH];
__shared__ uint4 g_p[H * PP];       // P as [head][8 chunks of 8 tokens], chunk ^ swz(head)
__shared__ float g_mx[2][H];
__shared__ int g_flag[4];

// Tile layout: 8-row x 8-chunk blocks of 1 KB; block (r/8, c/8) is block
// number (r/8)*9 + c/8 and row r%8 of it holds the row's 8 chunks permuted
// by XOR with swz(r), a permutation of (r/2)%8 whose values for rows r and
// r+2 (r%4 < 2) differ in bit 2. Sixteen consecutive rows at one chunk (one
// phase of the S fragment reads) and 4 rows x 4 chunks (one 32-lane phase of
// the transposed V reads) then fall on distinct banks.
__device__ __forceinline__ int swz(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int slot(int r, int c) {
  return ((r >> 3) * 9 + (c >> 3)) * 64 + (r & 7) * 8 + ((c & 7) ^ swz(r));
}

// Gather of one tile into `dst`: wave w loads rows 16w .. 16w+15 as 18
// direct-to-LDS instructions, each filling one 1 KB block (8 rows x 128
// bytes; lane l takes row r = 8*rg + l/8 and its logical chunk
// 8*ln + ((l%8) ^ swz(r)), so 8 adjacent lanes read one 128-byte line).
// The instructions are issued one by one between matrix-core operations:
// the address unit processes them at a fixed rate per CU, and issued in one
// burst they would stall the wave.
struct Gather {
  const uint16_t* src[2];
  __device__ __forceinline__ void setup(const uint16_t* kvb, int64_t kst, int ids, int w, int l) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int r = 8 * (2 * w + k) + (l >> 3);
      const int id = __shfl(ids, r, kWave);
      src[k] = kvb + static_cast<int64_t>(id < 0 ? 0 : id) * kst + 8 * ((l & 7) ^ swz(r));
    }
  }
  __device__ __forceinline__ void issue(uint4* dst, int w, int j) const {
    const int k = j / 9, ln = j % 9;
    __builtin_amdgcn_global_load_lds((glb_ptr)(src[k] + 64 * ln),
                                     (lds_ptr)(dst + ((2 * w + k) * 9 + ln) * 64), 16, 0, 0);
  }
};

struct State {
  bf16x8 qf[KS];
  f32x16 o[8];
  float m_run, l_run;
  bool seen;  // a valid token was seen (same in every wave: ids are shared)
};

// Reference maximum handling (base-2 logits, scale folded in): P of a tile
// is exponentiated against the reference agreed so far, so the two waves
// sharing a head need no exchange before the exponentials. Tile maxima are
// exchanged with P at the one barrier before P.V; afterwards the reference
// moves (and O, l are rescaled) when a tile maximum exceeds it by more than
// kLazy. Only the first valid tile, and a tile whose maximum exceeds the
// reference by more than kRedo (p would leave the fp32 range), take a second
// barrier and exponentiate against the exchanged maximum.
constexpr float kLazy = 8.0f, kRedo = 64.0f;

// One tile: S^T, softmax, P, O^T update. `cur` holds the tile; the next
// tile's gather into `nxt` is interleaved with the S products (always issued:
// past the last tile every id is -1 and the loads fetch row 0 again, which
// hits in cache), so the code is straight-line and the compiler's
// load-counter waits stay exact.
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
  const int jraw = tix[min(idx, topk - 1)];
  Gather ga;
  ga.setup(kvb, kst, ids_next, w, l);
  ids_cur = ids_next;
  ids_next = (idx < topk && jraw >= 0 && jraw < L) ? jraw : -1;

  // ---- S^T[tokens 32tt + (0..31)][heads 32hh + (0..31)] = K Q^T; each
  // fragment read is issued four MFMAs ahead of its use, and one gather
  // instruction of the next tile follows every second MFMA
  f32x16 sacc;
#pragma unroll
  for (int e = 0; e < 16; ++e) sacc[e] = 0.0f;
  {
    const int r = 32 * tt + l32;
    const unsigned char* tb = reinterpret_cast<const unsigned char*>(cur);
    int base[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) base[x] = 16 * slot(r, 2 * x + lh);
    uint4 kf[KS];
    constexpr int AHEAD = 4;
#pragma unroll
    for (int s = 0; s < AHEAD; ++s)
      kf[s] = *reinterpret_cast<const uint4*>(tb + base[s & 3] + 1024 * (s >> 2));
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if (s + AHEAD < KS)
        kf[s + AHEAD] =
            *reinterpret_cast<const uint4*>(tb + base[(s + AHEAD) & 3] + 1024 * ((s + AHEAD) >> 2));
      sacc = mfma32(as_bf16x8(kf[s]), st.qf[s], sacc);
      if (s & 1) ga.issue(nxt, w, s >> 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // ---- softmax over the tile (base 2, scale folded into the exponent)
  float sv[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) sv[e] = sacc[e];
  if (vmask != ~0ull) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int tk = 32 * tt + 8 * (e >> 2) + 4 * lh + (e & 3);
      if (!((vmask >> tk) & 1ull)) sv[e] = -INFINITY;
    }
  }
  float mloc = sv[0];
#pragma unroll
  for (int e = 1; e < 16; ++e) mloc = fmaxf(mloc, sv[e]);
  mloc = fmaxf(mloc, __shfl_xor(mloc, 32, kWave)) * scale_log2;
  if (lh == 0) g_mx[tt][head] = mloc;
  float mref = st.m_run;
  float mtile;
  const float l_prev = st.l_run;
  // exponentials of the tile against reference m; returns their sum and
  // writes P[head][token 32tt + 8q + 4lh + (0..3)] (chunk 4tt + q, half lh)
  auto make_p = [&](float m) -> float {
    const float mneg = m == -INFINITY ? 0.0f : -m;
    float ps = 0.0f;
    uint32_t pk[8];
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
      const float a = __builtin_amdgcn_exp2f(fmaf(sv[e], scale_log2, mneg));
      const float c = __builtin_amdgcn_exp2f(fmaf(sv[e + 1], scale_log2, mneg));
      ps += a + c;
      pk[e >> 1] = pack2(a, c);
    }
    uint2* prow = reinterpret_cast<uint2*>(g_p + head * PP);
#pragma unroll
    for (int qq = 0; qq < 4; ++qq)
      prow[2 * ((4 * tt + qq) ^ swz(head)) + lh] = make_uint2(pk[2 * qq], pk[2 * qq + 1]);
    return ps;
  };
  auto rescale_o = [&](float a) {
    if (__ballot(a != 1.0f) != 0ull) {
#pragma unroll
      for (int d = 0; d < 8; ++d)
#pragma unroll
        for (int e = 0; e < 16; ++e) st.o[d][e] *= a;
    }
  };
  if (!st.seen) {
    // no valid token seen before this tile (the same in every wave): agree
    // on the tile maximum first
    lds_barrier();
    mtile = fmaxf(mloc, g_mx[tt ^ 1][head]);
    mref = mtile;
    st.l_run = make_p(mref);
    lds_barrier();
  } else {
    g_flag[w] = __ballot(mloc > mref + kRedo) != 0ull ? 1 : 0;
    const float ps = make_p(mref);
    st.l_run = l_prev + ps;
    lds_barrier();
    mtile = fmaxf(mloc, g_mx[tt ^ 1][head]);
    if ((g_flag[0] | g_flag[1] | g_flag[2] | g_flag[3]) != 0) {
      // a score left the safe range above the reference: every wave redoes
      // the tile against the new maximum (S is still in registers)
      const float mnew = fmaxf(mref, mtile);
      const float alpha = __builtin_amdgcn_exp2f(mref - mnew);
      rescale_o(alpha);
      lds_barrier();  // everyone has read P and the maxima
      st.l_run = l_prev * alpha + make_p(mnew);
      mref = mnew;
      lds_barrier();
    }
  }
  st.m_run = mref;
  st.seen = st.seen || vmask != 0ull;

  // ---- O^T[dv 256tt + 32dt + (0..31)][heads] += V^T P^T over the tile's 64
  // tokens; V^T fragments (two transposed reads each) run three MFMAs ahead
  {
    const int G = l >> 4, sl = l & 15;
    const int trow = 8 * (G >> 1) + (sl >> 2);
    const int dcol = 16 * (G & 1) + 4 * (sl & 3);
    // row 16s + trow + 4h, chunk 32tt + 4dt + dcol/8: the s and dt/2 parts
    // are whole blocks (constant offsets), the rest one base per (h, dt&1)
    int vb[2][2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int dp = 0; dp < 2; ++dp)
        vb[h][dp] = 16 * slot(trow + 4 * h, 32 * tt + 4 * dp + (dcol >> 3)) + 2 * (dcol & 7);
    const unsigned char* tb = reinterpret_cast<const unsigned char*>(cur);
    auto vfrag = [&](int s, int dt) -> uint4 {
      const int off = s * 18 * 1024 + 1024 * (dt >> 1);
      const uint2 lo = tr16(tb + vb[0][dt & 1] + off);
      const uint2 hi = tr16(tb + vb[1][dt & 1] + off);
      return make_uint4(lo.x, lo.y, hi.x, hi.y);
    };
    bf16x8 pb[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) pb[s] = as_bf16x8(g_p[head * PP + ((2 * s + lh) ^ swz(head))]);
    constexpr int AHEAD = 3;
    uint4 vf[32];
#pragma unroll
    for (int i = 0; i < AHEAD; ++i) vf[i] = vfrag(i >> 3, i & 7);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if (i + AHEAD < 32) vf[i + AHEAD] = vfrag((i + AHEAD) >> 3, (i + AHEAD) & 7);
      st.o[i & 7] = mfma32(as_bf16x8(vf[i]), pb[i >> 3], st.o[i & 7]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // lazy move of the reference: the tile maximum (both token halves) is
  // known to every lane of a head, so all four copies decide alike
  const bool move = mtile > st.m_run + kLazy;
  if (__ballot(move) != 0ull) {
    const float a2 = move ? __builtin_amdgcn_exp2f(st.m_run - mtile) : 1.0f;
#pragma unroll
    for (int d = 0; d < 8; ++d)
#pragma unroll
      for (int e = 0; e < 16; ++e) st.o[d][e] *= a2;
    st.l_run *= a2;
    st.m_run = move ? mtile : st.m_run;
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
    // Q lives in AGPRs (the matrix cores read B operands from them directly),
    // leaving the VGPRs to the O accumulators and the fragment pipeline.
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      st.qf[s] = as_bf16x8(*reinterpret_cast<const uint4*>(qp + 16 * s));
      asm volatile("" : "+a"(st.qf[s]));
    }
  }
#pragma unroll
  for (int d = 0; d < 8; ++d) {
#pragma unroll
    for (int e = 0; e < 16; ++e) st.o[d][e] = 0.0f;
    asm volatile("" : "+v"(st.o[d]));
  }
  st.m_run = -INFINITY;
  st.l_run = 0.0f;
  st.seen = false;
  auto read_id = [&](int idx) -> int {
    const int j = tix[min(idx, topk - 1)];
    return (idx < topk && j >= 0 && j < L) ? j : -1;
  };
  int ids_cur = read_id(l);
  {
    Gather ga;
    ga.setup(kvb, ks.t, ids_cur, w, l);
#pragma unroll
    for (int j = 0; j < 18; ++j) ga.issue(g_tile_a, w, j);
  }
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
  float* lsum = reinterpret_cast<float*>(g_tile_b);   // tile memory is free now
  __syncthreads();
  if (lh == 0) lsum[tt * H + head] = lw;
  __syncthreads();
  const float ltot = lsum[head] + lsum[H + head];
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
