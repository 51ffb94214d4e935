// Sparse attention for multi-head latent attention rows: 64 query heads read
// one latent row per token of width 576, whose first 512 columns are also the
// value row. This is the shape of the 64K prefill workload and dominates its
// time (HISA explainer 1.1: attention over the selected tokens only; HISA
// news article: the downstream attention is unchanged).
//
// One workgroup of 8 waves per query, two per SIMD, in two roles:
//   * score waves (0..3), wave (hh, tt): heads 32hh..+32 and tokens 16tt..+16
//     of each tile. Their Q rows (32 heads x 576) stay in registers for the
//     whole query; S^T = K Q^T runs on 16x16x32 bf16 MFMA, then the softmax
//     numerators P = 2^(scale*log2(e)*S - R) go to LDS as bf16;
//   * value waves (4..7), wave 4+q: value columns 128q..+128 for all 64
//     heads. O^T = V^T P^T runs on 32x32x16 bf16 MFMA with O (64 x 128 fp32)
//     in registers; V^T fragments come straight from the row-major latent
//     tile through ds_read_tr16_b64, so V is never copied, and each fragment
//     feeds both 32-head halves. The value waves also move the data: they
//     read the token ids, publish each tile's validity mask and issue all
//     gathers.
// Each SIMD holds one wave of each role, so the softmax and the LDS waits of
// one overlap the matrix-core work of the other.
//
// The selected tokens stream through LDS in tiles of 32 latent rows (36 KB),
// four resident at once. In iteration i the score waves compute S(i) and P(i)
// while the value waves accumulate P(i-1) V(i-1) and gather tile i+2; one
// barrier per iteration. Gathers go HBM/L2 -> LDS with 16-byte direct loads
// (global_load_lds); the 16-byte chunks of each row are XOR-swizzled so every
// fragment read is free of bank conflicts (8 adjacent lanes still read one
// 128-byte line). Token ids take the same direct-load path into a ring in
// LDS, so the loop issues no other global loads and every load-counter wait
// covers exactly the loads it names. Workgroups are mapped so each XCD walks
// a contiguous range of queries: neighbouring queries share their forced
// blocks and sweep the same token range together, which raises L2 reuse.
//
// Softmax reference. Every head's numerators are taken against one reference
// R per query: the maximum over the first tile's valid tokens (base-2
// logits, scale folded in). A later score more than kRedo above R would let a
// numerator leave the safe range; the score wave that sees one raises a flag,
// and after the barrier every wave redoes that tile against the exchanged
// tile maximum (rescaling the partial sums and O). Numerators far below R
// underflow to zero, which is exact to fp32 since R never exceeds the true
// maximum. With kRedo = 64 the fp32 sums stay below 2^64 * 2^14 per head.
//
// The last two iterations gather nothing (there is no tile past the end),
// and the value waves store the normalised O straight from registers, so a
// workgroup's end overlaps little with the start of the next one on its CU.
#include <algorithm>
#include <cstdlib>

#include "common.hpp"
#include "internal.h"

namespace hisa {
namespace mla {

constexpr int H = 64, DK = 576, DV = 512;
constexpr int NT = 32;          // tokens per tile
constexpr int RCH = DK / 8;     // 16-byte chunks per latent row (72)
constexpr int TCH = NT * RCH;   // chunk slots per tile (2304 = 36 KB)
constexpr int KS = DK / 32;     // k steps of S (18)
constexpr int PCH = NT / 8;     // 16-byte chunks per P row (4)
constexpr int NBLK = RCH / 8;   // 1 KB blocks per 8-row group (9)
constexpr float kRedo = 64.0f;
constexpr int kRotTicks = 96;   // clock ticks per tile of the rotated sweep (measured best)

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
// Reductions over the lane groups l, l^16, l^32, l^48 with the VALU row
// swaps: the pair of outputs of a swap holds this lane's row and its partner's.
__device__ __forceinline__ float max_x16_x32(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_x16_x32(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
// LDS-only barrier: wait for this wave's LDS operations, then s_barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
}
__device__ __forceinline__ float exp2_ratio(float from, float to) {
  return from == to ? 1.0f : __builtin_amdgcn_exp2f(from - to);
}

__shared__ uint4 g_t0[TCH];
__shared__ uint4 g_t1[TCH];
__shared__ uint4 g_t2[TCH];
__shared__ uint4 g_t3[TCH];
__shared__ uint4 g_p0[H * PCH];     // P as [head][4 chunks of 8 tokens]
__shared__ uint4 g_p1[H * PCH];
__shared__ float g_mx[2][H];        // tile maxima per token half (first tile and redo only)
__shared__ int g_flag0[4];          // redo flags per score wave, even / odd tiles
__shared__ int g_flag1[4];
__shared__ uint32_t g_mask[2];      // valid-token masks, even / odd tiles
__shared__ int g_ids[8][64];        // token ids of eight tiles (ring; lanes 32..63 repeat)

template <int I>
__device__ __forceinline__ uint4* tbuf() {
  if constexpr ((I & 3) == 0) return g_t0;
  else if constexpr ((I & 3) == 1) return g_t1;
  else if constexpr ((I & 3) == 2) return g_t2;
  else return g_t3;
}
template <int I>
__device__ __forceinline__ int* flagbuf() {
  if constexpr ((I & 1) == 0) return g_flag0;
  else return g_flag1;
}
template <int I>
__device__ __forceinline__ uint4* pbuf() {
  if constexpr ((I & 1) == 0) return g_p0;
  else return g_p1;
}

// Tile layout: 8-row x 8-chunk blocks of 1 KB; block (r/8, c/8) is block
// number (r/8)*9 + c/8 and row r%8 of it holds the row's 8 chunks permuted
// by XOR with swz(r), which swaps bits 1 and 2 of r (bit 0 and bit 3 drop
// out). The LDS serves a 16-byte read 16 lanes at a time, the lanes of one
// cycle being the four lane quads whose quad index (lane bits 2..4) has one
// parity, within each 32-lane half; it serves a transposing 8-byte read 32
// lanes at a time. With this swizzle the 16 lanes of each cycle of an S
// fragment read (16 rows at two adjacent chunks) and the 32 lanes of each
// cycle of a transposed V read (4 rows x 4 chunks) fall on distinct banks.
__device__ __forceinline__ int swz(int r) { return ((r & 4) >> 1) | ((r & 2) << 1); }
__device__ __forceinline__ int slot(int r, int c) {
  return ((r >> 3) * 9 + (c >> 3)) * 64 + (r & 7) * 8 + ((c & 7) ^ swz(r));
}
// P row h holds tokens 0..31 as 4 chunks, chunk c at position c ^ ((h/4)%4):
// 16 consecutive heads at one chunk cover all 64 banks.
__device__ __forceinline__ int pslot(int h, int c) { return h * PCH + (c ^ ((h >> 2) & 3)); }

// Ids outside [0, L) (padding, or past the end of the list) load row 0; such
// tokens are masked out of the softmax. Iteration `it` reads list tile
// `tile` into ring slot it % 8.
__device__ __forceinline__ void ids_issue(const int32_t* tix, int topk, int it, int tile, int l) {
  __builtin_amdgcn_global_load_lds((glb_ptr)(tix + min(tile * NT + (l & 31), topk - 1)),
                                   (lds_ptr)(&g_ids[it & 7][0]), 4, 0, 0);
}
__device__ __forceinline__ uint32_t id_addr(int tile, int t) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) int*)(&g_ids[tile & 7][t]);
}
// Two ids (tile a, token ta) and (tile b, token tb) per lane. Ids are loaded
// several tiles ahead and are covered by an earlier barrier's load-counter
// wait; the reads are written out here because the compiler cannot tell the
// ring slots apart and would otherwise drain every load in flight first. The
// wait also covers any LDS read the caller issued just before.
__device__ __forceinline__ int2 read_ids(int tile_a, int ta, int tile_b, int tb) {
  int a, b;
  asm volatile("ds_read_b32 %0, %2\n\tds_read_b32 %1, %3\n\ts_waitcnt lgkmcnt(0)"
               : "=&v"(a), "=&v"(b)
               : "v"(id_addr(tile_a, ta)), "v"(id_addr(tile_b, tb))
               : "memory");
  return make_int2(a, b);
}
__device__ __forceinline__ uint32_t tile_mask(int id, int topk, int L, int tile, int l) {
  return static_cast<uint32_t>(__ballot(tile * NT + (l & 31) < topk &&
                                        static_cast<unsigned>(id) < static_cast<unsigned>(L)));
}
// Gather of one tile's row group rg (rows 8rg .. 8rg+7) as 9 blocks of 1 KB
// (8 rows x 128 bytes); one direct-to-LDS instruction fills a block, lane l
// taking row r = 8rg + l/8 and its logical chunk 8*ln + ((l%8) ^ swz(r)), so
// 8 adjacent lanes read one 128-byte line. The instructions are spread
// between matrix-core operations: the address unit processes them at a fixed
// rate per CU, and issued in one burst they would stall the wave.
// id: the id of row r = 8rg + l/8 of the tile
__device__ __forceinline__ const uint16_t* gather_src(const uint16_t* kvb, int64_t kst, int L,
                                                      int id, int rg, int l) {
  const int r = 8 * rg + (l >> 3);
  const int row = static_cast<unsigned>(id) < static_cast<unsigned>(L) ? id : 0;
  return kvb + static_cast<int64_t>(row) * kst + 8 * ((l & 7) ^ swz(r));
}
__device__ __forceinline__ void gather_issue(const uint16_t* src, uint4* dst, int rg, int ln) {
  __builtin_amdgcn_global_load_lds((glb_ptr)(src + 64 * ln), (lds_ptr)(dst + (rg * NBLK + ln) * 64),
                                   16, 0, 0);
}

struct Ctx {
  const uint16_t* kvb;
  int64_t kst;
  const int32_t* tix;
  int topk, L;
  float scale_log2, inv_scale_log2;
  int w;
  int first, ntiles;  // the list tile of iteration 0, the list's tiles
  // list tile of iteration i: the tiles in cyclic order from `first`; the
  // padding iterations past the list keep their own index (fully masked)
  __device__ __forceinline__ int tile(int i) const {
    if (i >= ntiles) return i;
    const int t = first + i;
    return t < ntiles ? t : t - ntiles;
  }
};

// ------------------------------------------------------------- score waves
struct SState {
  bf16x8 qf[2][KS];         // Q fragments of heads 32hh + 16hb + (0..15)
  f32x4 s[2];               // S of the current tile (masked in place)
  float R[2];               // reference of heads 32hh + 16hb + l%16
  float lsum[2], lprev[2];  // partial row sums over this wave's tokens
};

// Numerators of head block hb against reference m into P (tile parity I) at
// tokens 16tt + 4g + (0..3); returns their sum. The stores of the two head
// blocks are kept apart (separately computed addresses, a scheduling fence
// between the calls): merged, or folded into one base plus an offset, they
// lose the information that tells them apart from the tile loads in flight,
// and the compiler would wait for all of those first.
template <int I>
__device__ __forceinline__ float make_p(const SState& st, int hb, float m, float scale_log2, int hh,
                                        int tt, int l) {
  const float mneg = m == -INFINITY ? 0.0f : -m;
  float p[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) p[r] = __builtin_amdgcn_exp2f(fmaf(st.s[hb][r], scale_log2, mneg));
  int hoff = 16 * hb;
  asm volatile("" : "+v"(hoff));
  const int h = 32 * hh + hoff + (l & 15);
  const int g = l >> 4;
  unsigned char* prow = reinterpret_cast<unsigned char*>(pbuf<I>());
  *reinterpret_cast<uint2*>(prow + 16 * pslot(h, 2 * tt + (g >> 1)) + 8 * (g & 1)) =
      make_uint2(pack2(p[0], p[1]), pack2(p[2], p[3]));
  return (p[0] + p[1]) + (p[2] + p[3]);
}

// This wave's maximum (base 2) of head block hb over its 16 tokens of S,
// published for the partner score wave of the same heads.
__device__ __forceinline__ void publish_max(const SState& st, int hb, float scale_log2, int hh,
                                            int tt, int l) {
  const float m = max_x16_x32(fmaxf(fmaxf(st.s[hb][0], st.s[hb][1]),
                                    fmaxf(st.s[hb][2], st.s[hb][3]))) * scale_log2;
  if ((l >> 4) == 0) g_mx[tt][32 * hh + 16 * hb + (l & 15)] = m;
}

// After the barrier that follows tile j (parity J): if any score wave flagged
// tile j, exchange its maxima and redo P(j) against them (two barriers, taken
// by every wave alike).
template <int J>
__device__ __forceinline__ void s_settle(SState& st, const Ctx& cx, int hh, int tt, int l) {
  const int* fl = flagbuf<J>();
  const int any = __builtin_amdgcn_readfirstlane(fl[0] | fl[1] | fl[2] | fl[3]);
  if (any != 0) {
    publish_max(st, 0, cx.scale_log2, hh, tt, l);
    publish_max(st, 1, cx.scale_log2, hh, tt, l);
    lds_barrier();
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int h = 32 * hh + 16 * hb + (l & 15);
      const float mnew = fmaxf(st.R[hb], fmaxf(g_mx[0][h], g_mx[1][h]));
      const float a = exp2_ratio(st.R[hb], mnew);
      st.lsum[hb] = st.lprev[hb] * a + make_p<J>(st, hb, mnew, cx.scale_log2, hh, tt, l);
      st.R[hb] = mnew;
      __builtin_amdgcn_sched_barrier(0);
    }
    lds_barrier();
  }
}

// Score wave, iteration i (I = i mod 4): settle tile i-1, S(i), numerators
// of S(i) into P(i), barrier.
template <int I, bool FIRST>
__device__ __forceinline__ void s_iter(SState& st, const Ctx& cx, int l) {
  const int w = cx.w, hh = w >> 1, tt = w & 1;
  if constexpr (!FIRST) s_settle<I + 3>(st, cx, hh, tt, l);
  const uint32_t vmask = g_mask[I & 1];

  // ---- S^T[tokens 16tt + (0..15)][heads 32hh + 16hb + (0..15)] of tile i
  f32x4 acc[2];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[hb][e] = 0.0f;
  {
    const int r = 16 * tt + (l & 15), g = l >> 4;
    const unsigned char* tb = reinterpret_cast<const unsigned char*>(tbuf<I>());
    int base[2];
#pragma unroll
    for (int x = 0; x < 2; ++x) base[x] = 16 * slot(r, 4 * x + g);
    auto kfrag = [&](int s) -> uint4 {
      return *reinterpret_cast<const uint4*>(tb + base[s & 1] + 1024 * (s >> 1));
    };
    constexpr int AHEAD = 4;
    uint4 kf[KS];
#pragma unroll
    for (int s = 0; s < AHEAD; ++s) kf[s] = kfrag(s);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if (s + AHEAD < KS) kf[s + AHEAD] = kfrag(s + AHEAD);
      acc[0] = mfma16(as_bf16x8(kf[s]), st.qf[0][s], acc[0]);
      acc[1] = mfma16(as_bf16x8(kf[s]), st.qf[1][s], acc[1]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  st.s[0] = acc[0];
  st.s[1] = acc[1];

  // ---- numerators of tile i
  if (vmask != 0xFFFFFFFFu) {
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tk = 16 * tt + 4 * (l >> 4) + r;
        if (!((vmask >> tk) & 1u)) st.s[hb][r] = -INFINITY;
      }
  }
  if constexpr (FIRST) {
    // the reference: the first tile's maximum, agreed between the partners
    publish_max(st, 0, cx.scale_log2, hh, tt, l);
    publish_max(st, 1, cx.scale_log2, hh, tt, l);
    lds_barrier();
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int h = 32 * hh + 16 * hb + (l & 15);
      st.R[hb] = fmaxf(g_mx[0][h], g_mx[1][h]);
    }
  }
  bool flag = false;
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const float lim = (st.R[hb] + kRedo) * cx.inv_scale_log2;  // in units of S
#pragma unroll
    for (int r = 0; r < 4; ++r) flag = flag || st.s[hb][r] > lim;
  }
  const bool any = __ballot(flag) != 0ull;
  if (l == 0) flagbuf<I>()[w] = any ? 1 : 0;
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    st.lprev[hb] = st.lsum[hb];
    st.lsum[hb] += make_p<I>(st, hb, st.R[hb], cx.scale_log2, hh, tt, l);
    __builtin_amdgcn_sched_barrier(0);
  }
  lds_barrier();
}

// ------------------------------------------------------------- value waves
struct VState {
  f32x16 o[8];              // O^T accumulators, index 2*dt + hb
  float ro[2];              // reference of heads 32hb + l%32 (the scale of O)
  const uint16_t* gsrc;     // gather source of the tile being loaded
};

__device__ __forceinline__ void scale_in_place(f32x16& o, float a) {
#pragma unroll
  for (int e = 0; e < 16; ++e) asm volatile("v_mul_f32 %0, %1, %0" : "+v"(o[e]) : "v"(a));
}

// The value-wave side of the settle (same flags, same two barriers): take
// the raised reference and bring O to it. The products are written in place
// (tied operands) so the accumulators keep their registers.
template <int J>
__device__ __forceinline__ void v_settle(VState& st, int any, int l) {
  if (any != 0) {
    lds_barrier();
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int h = 32 * hb + (l & 31);
      const float mnew = fmaxf(st.ro[hb], fmaxf(g_mx[0][h], g_mx[1][h]));
      const float a = exp2_ratio(st.ro[hb], mnew);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) scale_in_place(st.o[2 * dt + hb], a);
      st.ro[hb] = mnew;
    }
    lds_barrier();
  }
}

// The data movement of iteration i: the gather source of tile i+2, the mask
// of tile i+1 (published for the score waves), the ids of tile i+5. Returns
// the redo flags of tile i-1 (parity J), read in the same LDS round trip.
template <int J>
__device__ __forceinline__ int v_ids(VState& st, const Ctx& cx, int i, int q4, int l) {
  const int4 fl = *reinterpret_cast<const int4*>(flagbuf<J>());
  const int2 id = read_ids(i + 2, 8 * q4 + (l >> 3), i + 1, l & 31);
  st.gsrc = gather_src(cx.kvb, cx.kst, cx.L, id.x, q4, l);
  const uint32_t m = tile_mask(id.y, cx.topk, cx.L, cx.tile(i + 1), l);
  if (q4 == 0 && l == 0) g_mask[(i + 1) & 1] = m;
  __builtin_amdgcn_sched_barrier(0);
  ids_issue(cx.tix, cx.topk, i + 5, cx.tile(i + 5), l);
  __builtin_amdgcn_sched_barrier(0);
  return __builtin_amdgcn_readfirstlane(fl.x | fl.y | fl.z | fl.w);
}

// O^T[dv 128q4 + 32dt + (0..31)][heads 32hb + (0..31)] += V^T P^T over the
// tile of parity J; with GATHER, the 9 blocks of the tile being loaded are
// issued between the matrix-core operations
template <int J, bool GATHER>
__device__ __forceinline__ void v_accumulate(VState& st, int q4, int l, uint4* gdst) {
  // The fragment addresses derived from the lane id stay in registers across
  // the loop (216 VGPRs, still two waves per SIMD).
  bf16x8 pb[2][2];
  {
    const uint4* pp = pbuf<J>();
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        pb[hb][ks] = as_bf16x8(pp[pslot(32 * hb + (l & 31), 2 * ks + (l >> 5))]);
  }
  // V^T fragment (ks, dt): rows 16ks + trow + 4h, chunk 16q4 + 4dt + dcol/8
  const int G = l >> 4, sl = l & 15;
  const int trow = 8 * (G >> 1) + (sl >> 2);
  const int dcol = 16 * (G & 1) + 4 * (sl & 3);
  int vb[2][2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int dp = 0; dp < 2; ++dp)
      vb[h][dp] = 16 * slot(trow + 4 * h, 16 * q4 + 4 * dp + (dcol >> 3)) + 2 * (dcol & 7);
  const unsigned char* tb = reinterpret_cast<const unsigned char*>(tbuf<J>());
  auto vfrag = [&](int ks, int dt) -> uint4 {
    const int off = ks * 18 * 1024 + 1024 * (dt >> 1);
    const uint2 lo = tr16(tb + vb[0][dt & 1] + off);
    const uint2 hi = tr16(tb + vb[1][dt & 1] + off);
    return make_uint4(lo.x, lo.y, hi.x, hi.y);
  };
  constexpr int AHEAD = 4;
  uint4 vf[8];
#pragma unroll
  for (int x = 0; x < AHEAD; ++x) vf[x] = vfrag(x >> 2, x & 3);
#pragma unroll
  for (int x = 0; x < 8; ++x) {
    if (x + AHEAD < 8) vf[x + AHEAD] = vfrag((x + AHEAD) >> 2, (x + AHEAD) & 3);
    const int ks = x >> 2, dt = x & 3;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      st.o[2 * dt + hb] = mfma32(as_bf16x8(vf[x]), pb[hb][ks], st.o[2 * dt + hb]);
      if constexpr (GATHER) {
        if (hb == 0) gather_issue(st.gsrc, gdst, q4, x);
        else if (x == 7) gather_issue(st.gsrc, gdst, q4, 8);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Value wave, iteration i: settle tile i-1, the data movement, O += P(i-1)
// V(i-1) with the gathers of tile i+2 interleaved, barrier.
template <int I, bool FIRST, bool GATHER = true>
__device__ __forceinline__ void v_iter(VState& st, const Ctx& cx, int i, int l) {
  const int q4 = cx.w - 4;
  const int any = v_ids<I + 3>(st, cx, i, q4, l);
  if constexpr (!FIRST) v_settle<I + 3>(st, any, l);
  if constexpr (FIRST) {
#pragma unroll
    for (int ln = 0; ln < NBLK; ++ln) gather_issue(st.gsrc, tbuf<I + 2>(), q4, ln);
    // the score waves agree on the reference
    lds_barrier();
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int h = 32 * hb + (l & 31);
      st.ro[hb] = fmaxf(g_mx[0][h], g_mx[1][h]);
    }
  } else {
    v_accumulate<I + 3, GATHER>(st, q4, l, tbuf<I + 2>());
  }
  // tile i+1 is complete once at most this iteration's loads (the ids of
  // tile i+5 and, but in the last two iterations, the 9 gather blocks of
  // tile i+2) are outstanding
  if constexpr (GATHER) __builtin_amdgcn_s_waitcnt(0x007A);  // vmcnt(10) lgkmcnt(0)
  else __builtin_amdgcn_s_waitcnt(0x0071);                    // vmcnt(1) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
}

__shared__ int g_first;          // the list tile of iteration 0

__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mla_attn_kernel(const uint16_t* __restrict__ q, Str3 qs, const uint16_t* __restrict__ kv,
                     Str3 ks, int nq, int L, int Hkv, const int32_t* __restrict__ token_idx,
                     int topk, float scale_log2, uint16_t* __restrict__ out, Str3 os,
                     float* __restrict__ lse, int rot_ticks) {
  const int per = (nq + 7) / 8;
  const int qi = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (qi >= nq) return;
  const int b = blockIdx.y / Hkv, g = blockIdx.y % Hkv;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
  const int64_t qrow = static_cast<int64_t>(b) * nq + qi;
  const int32_t* tix = token_idx + qrow * topk;
  const int ntiles = (topk + NT - 1) / NT;
  const int nt4 = (ntiles + 3) & ~3;  // tiles processed: a multiple of 4, extra ones fully masked
  // Sweep order. With rot_ticks > 0 the query starts at list tile
  // (clock / rot_ticks) mod ntiles and wraps around: every query in flight
  // then reads the same part of its ascending list (the same region of the
  // cache) at the same time, whenever it started, so rows that neighbouring
  // queries share are fetched into L2 once. The softmax is the same for any
  // order (the reference comes from the first tile processed); only the fp32
  // summation order follows the clock. One clock read per workgroup, shared.
  if (tid == 0)
    g_first = rot_ticks > 0
                  ? static_cast<int>((__builtin_amdgcn_s_memrealtime() / rot_ticks) % ntiles)
                  : 0;
  __syncthreads();

  Ctx cx;
  cx.kvb = kv + b * ks.b + g * ks.h;
  cx.kst = ks.t;
  cx.tix = tix;
  cx.topk = topk;
  cx.L = L;
  cx.scale_log2 = scale_log2;
  cx.inv_scale_log2 = 1.0f / scale_log2;
  cx.w = w;
  cx.first = __builtin_amdgcn_readfirstlane(g_first);
  cx.ntiles = ntiles;

  float* lsum_x = &g_mx[0][0];  // reused after the loop for the row sums
  if (w < 4) {
    // ================================================= score waves
    const int hh = w >> 1, tt = w & 1;
    SState st;
    {
      // Q fragments of heads 32hh + 16hb + l%16, k chunk 4s + l/16
      const uint16_t* qp =
          q + b * qs.b + qi * qs.t + (g * H + 32 * hh + (l & 15)) * qs.h + 8 * (l >> 4);
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int s = 0; s < KS; ++s)
          st.qf[hb][s] = as_bf16x8(*reinterpret_cast<const uint4*>(qp + 16 * hb * qs.h + 32 * s));
    }
    st.R[0] = st.R[1] = -INFINITY;
    st.lsum[0] = st.lsum[1] = st.lprev[0] = st.lprev[1] = 0.0f;
    __builtin_amdgcn_s_waitcnt(0x0070);  // Q has arrived
    __builtin_amdgcn_s_barrier();        // tile 0 and its mask are resident
    s_iter<0, true>(st, cx, l);
    int i = 1;
    for (; i + 3 < nt4; i += 4) {
      s_iter<1, false>(st, cx, l);
      s_iter<2, false>(st, cx, l);
      s_iter<3, false>(st, cx, l);
      s_iter<0, false>(st, cx, l);
    }
    s_iter<1, false>(st, cx, l);
    s_iter<2, false>(st, cx, l);
    s_iter<3, false>(st, cx, l);
    s_settle<3>(st, cx, hh, tt, l);  // the last tile (nt4-1)
    const float l0 = sum_x16_x32(st.lsum[0]);
    const float l1 = sum_x16_x32(st.lsum[1]);
    __syncthreads();
    if ((l >> 4) == 0) {
      lsum_x[tt * H + 32 * hh + (l & 15)] = l0;
      lsum_x[tt * H + 32 * hh + 16 + (l & 15)] = l1;
    }
    __syncthreads();
  } else {
    // ================================================= value waves
    const int q4 = w - 4;
    VState st;
#pragma unroll
    for (int t = 0; t < 5; ++t) ids_issue(tix, topk, t, cx.tile(t), l);
#pragma unroll
    for (int d = 0; d < 8; ++d) {
#pragma unroll
      for (int e = 0; e < 16; ++e) st.o[d][e] = 0.0f;
    }
    st.ro[0] = st.ro[1] = -INFINITY;
    __builtin_amdgcn_s_waitcnt(0x0070);  // the ids of tiles 0..4 have arrived
    {
      const int2 id = read_ids(0, 8 * q4 + (l >> 3), 1, 8 * q4 + (l >> 3));
      const int2 idm = read_ids(0, l & 31, 0, l & 31);
      const uint32_t m0 = tile_mask(idm.x, topk, L, cx.tile(0), l);
      if (q4 == 0 && l == 0) g_mask[0] = m0;
      const uint16_t* s0 = gather_src(cx.kvb, cx.kst, L, id.x, q4, l);
#pragma unroll
      for (int ln = 0; ln < NBLK; ++ln) gather_issue(s0, g_t0, q4, ln);
      const uint16_t* s1 = gather_src(cx.kvb, cx.kst, L, id.y, q4, l);
#pragma unroll
      for (int ln = 0; ln < NBLK; ++ln) gather_issue(s1, g_t1, q4, ln);
    }
    __builtin_amdgcn_s_waitcnt(0x0079);  // vmcnt(9) lgkmcnt(0): tile 0 is resident
    __builtin_amdgcn_s_barrier();
    v_iter<0, true>(st, cx, 0, l);
    int i = 1;
    for (; i + 3 < nt4; i += 4) {
      v_iter<1, false>(st, cx, i, l);
      v_iter<2, false>(st, cx, i + 1, l);
      v_iter<3, false>(st, cx, i + 2, l);
      v_iter<0, false>(st, cx, i + 3, l);
    }
    v_iter<1, false>(st, cx, i, l);
    v_iter<2, false, false>(st, cx, i + 1, l);  // tiles i+3 = nt4 and nt4+1 do not exist
    v_iter<3, false, false>(st, cx, i + 2, l);
    // the last tile (nt4-1, parity 3)
    {
      const int* fl = flagbuf<3>();
      v_settle<3>(st, __builtin_amdgcn_readfirstlane(fl[0] | fl[1] | fl[2] | fl[3]), l);
    }
    v_accumulate<3, false>(st, q4, l, nullptr);
    __builtin_amdgcn_s_waitcnt(0x0070);  // the ids loaded past the end
    __syncthreads();
    // (the score waves write the row sums here)
    __syncthreads();
    // ---- normalise O and store it from registers. Lane l holds head
    // 32hb + l%32 and, per 32-column block, the columns 8i + 4(l/32) + (0..3);
    // one swap across the lane halves gives every lane 8 consecutive columns.
    uint16_t* orow = out + b * os.b + qi * os.t + g * H * os.h;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int h = 32 * hb + (l & 31);
      const float ltot = lsum_x[h] + lsum_x[H + h];
      const float inv = ltot > 0.0f ? 1.0f / ltot : 0.0f;
      if (lse != nullptr && q4 == 0 && (l >> 5) == 0)
        lse[qrow * (static_cast<int64_t>(H) * Hkv) + g * H + h] =
            ltot > 0.0f ? (st.ro[hb] + log2f(ltot)) * 0.69314718055994530942f : -INFINITY;
      uint16_t* op = orow + static_cast<int64_t>(h) * os.h + 128 * q4 + 8 * ((l >> 5) ^ 1);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const f32x16& o = st.o[2 * dt + hb];
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
          // quads 2pr (columns 16pr + 4(l/32) + (0..3)) and 2pr+1 (+8)
          const int e0 = 8 * pr, e1 = 8 * pr + 4;
          const uint32_t x0 = pack2(o[e1 + 0] * inv, o[e1 + 1] * inv);
          const uint32_t x1 = pack2(o[e1 + 2] * inv, o[e1 + 3] * inv);
          const uint32_t y0 = pack2(o[e0 + 0] * inv, o[e0 + 1] * inv);
          const uint32_t y1 = pack2(o[e0 + 2] * inv, o[e0 + 3] * inv);
          const auto s0 = __builtin_amdgcn_permlane32_swap(x0, y0, false, false);
          const auto s1 = __builtin_amdgcn_permlane32_swap(x1, y1, false, false);
          // lanes < 32: columns 16pr + 8 .. +15; lanes >= 32: 16pr + 0 .. +7
          *reinterpret_cast<uint4*>(op + 32 * dt + 16 * pr) =
              make_uint4(s0[0], s1[0], s0[1], s1[1]);
        }
      }
    }
  }
}

}  // namespace mla

// The clock period (ticks of the 100 MHz real-time counter) per tile of the
// rotated sweep; HISA_MLA_ROT_TICKS overrides it, 0 giving the list order
// (bit-reproducible outputs).
static int mla_rot_ticks() {
  const char* e = getenv("HISA_MLA_ROT_TICKS");
  if (e != nullptr && *e != '\0') return std::max(0, atoi(e));
  return mla::kRotTicks;
}

hipError_t launch_mla_attn(const uint16_t* q, Str3 qs, const uint16_t* kv, Str3 ks, int batch,
                           int nq, int L, int Hkv, const int32_t* token_idx, int topk, float scale,
                           uint16_t* out, Str3 os, float* lse, hipStream_t s) {
  const int per = (nq + 7) / 8;
  hipLaunchKernelGGL(mla::mla_attn_kernel, dim3(8 * per, batch * Hkv), dim3(512), 0, s, q, qs,
                     kv, ks, nq, L, Hkv, token_idx, topk, scale * 1.44269504088896340736f, out,
                     os, lse, mla_rot_ticks());
  return hipGetLastError();
}

}  // namespace hisa
