// Sparse attention over the selected tokens for head width 128 (Dk = Dv =
// 128) and at most 16 query heads per kv head: the MQA prefill (16 heads over
// one kv head), the decode batch and the small prefill (HISA explainer 1.1:
// attention over the selected tokens only; HISA news article: the downstream
// attention is unchanged).
//
// One wave per (sequence, query, kv head), two independent waves per
// workgroup, no workgroup barrier. The kept tokens stream through the wave's
// own LDS ring of two 16-token tiles (K and V, 4 KB each), gathered
// HBM/L2 -> LDS with 16-byte direct loads two tiles ahead: a tile's K and V
// fragments are all read into registers under one wait before the gathers
// of the tile two ahead are issued into the same slot, so two slots carry a
// two-tile prefetch (18 KB of LDS per wave, eight waves per CU). Token ids
// take the same path into a ring of their own, so the loop issues no other
// global load and each load-counter wait covers exactly the loads it names.
//
// Per tile: S^T = K Q^T on 16x16x32 bf16 MFMA (K fragments from LDS, the
// group's Q rows in registers). Its accumulator holds, in lane l, head l%16
// and tokens 4(l/16)..+3, the A operand layout of a 16x16x16 MFMA, so the
// numerators P feed O += P V without passing through LDS; V^T fragments come
// from the row-major V tile through ds_read_tr16_b64. The products of two
// consecutive tiles run together as 16x16x32 MFMAs (each lane's 4 tokens of
// both tiles as its 8 k values).
//
// Softmax reference: R per head is the maximum over the query's first tile's
// valid tokens (base-2 logits, scale folded in); a later tile whose maximum
// exceeds R by more than kRaise raises R to it, rescaling the row sums and O
// (rare). Numerators far below R underflow to zero, exact to fp32 since R
// never exceeds the true maximum; no numerator exceeds 2^64.
//
// Few (query, kv head) pairs (decode) would leave most CUs idle, so their
// token lists are split: each wave takes a run of tiles and writes its O, R
// and row sums in fp32, and a second kernel rescales the splits to a common
// maximum and sums them.
#include <algorithm>

#include "common.hpp"
#include "internal.h"

namespace hisa {
namespace d128 {

constexpr int D = 128;
constexpr int NT = 16;             // tokens per tile
constexpr int TCH = NT * D / 8;    // 16-byte chunks per K or V tile (256)
constexpr int WAVES = 2;           // independent waves per workgroup
constexpr float kRaise = 64.0f;
constexpr int64_t kSplitWaves = 512;  // split the lists while fewer waves than this
constexpr int kMinSplitTiles = 4;      // tiles per split, at least

typedef __attribute__((address_space(3))) void* lds_ptr;
typedef __attribute__((address_space(1))) void* glb_ptr;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short v4s;

// The ring slots are separate objects (indexed by the wave), so a read of
// one slot is never mistaken for a read of the slot being gathered into.
__shared__ uint4 g_k0[WAVES][TCH];
__shared__ uint4 g_k1[WAVES][TCH];
__shared__ uint4 g_v0[WAVES][TCH];
__shared__ uint4 g_v1[WAVES][TCH];
__shared__ int g_ids[WAVES][8][64];  // ids of eight tiles (lanes 16..63 repeat)

// Slot of tile I (mod 2).
template <int I>
__device__ __forceinline__ uint4* kbuf(int w) {
  if constexpr (I % 2 == 0) return g_k0[w];
  else return g_k1[w];
}
template <int I>
__device__ __forceinline__ uint4* vbuf(int w) {
  if constexpr (I % 2 == 0) return g_v0[w];
  else return g_v1[w];
}

// Tile layout: row r (a token) holds its 16 chunks of 16 bytes permuted by
// XOR with swz(r). The LDS serves a 16-byte read 16 lanes at a time (the
// four lane quads whose quad index has one parity, within each 32-lane half)
// and a transposing 8-byte read 32 lanes at a time; with this swizzle both
// the K fragment reads (16 rows at one chunk) and the V^T reads (4 rows x 32
// bytes per 16 lanes) fall on distinct banks.
__device__ __forceinline__ int swz(int r) { return ((r & 7) << 1) ^ (r & 8); }

__device__ __forceinline__ f32x4 mfma16k16(const v4s& a, const v4s& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
// The larger of two scores. Written out: fmaxf first quiets each operand
// (one extra instruction per operand), and no score is a NaN.
__device__ __forceinline__ float vmax(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float max_x16_x32(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  v = vmax(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return vmax(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_x16_x32(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ float exp2_ratio(float from, float to) {
  return from == to ? 1.0f : __builtin_amdgcn_exp2f(from - to);
}

struct Item {
  const uint16_t* kb;   // K rows of this kv head
  const uint16_t* vb;   // V rows of this kv head
  const int32_t* tix;   // this query's token ids
  int64_t kst, vst;     // row strides (elements)
  uint32_t kbytes, vbytes;  // row strides in bytes (32-bit offset form)
  int topk, L, w;
};

// Ids of tile t into ring slot t % 8: lane p < 16 loads id 4(p%4) + p/4 of
// the tile, so the four ids a gather lane needs (rows 4u + g, u = 0..3, for
// its lane group g) sit next to each other. Ids past the list repeat the last
// one; such tokens are masked.
__device__ __forceinline__ void ids_issue(const Item& it, int t, int l) {
  const int p = l & 15;
  const int j = min(NT * t + 4 * (p & 3) + (p >> 2), it.topk - 1);
  __builtin_amdgcn_global_load_lds((glb_ptr)(it.tix + j), (lds_ptr)(&g_ids[it.w][t & 7][0]), 4, 0,
                                   0);
}
// The four ids of this lane's gather rows for tile t (landed by an earlier
// load-counter wait). Written out because the compiler cannot tell the ring
// slots apart and would otherwise drain every load in flight first. The wait
// stays in the same statement as the read: the compiler takes an asm output
// as written when its statement ends, so after a read without its wait it may
// copy the destination registers before the data has arrived. The wait also
// covers every LDS read the wave issued before.
__device__ __forceinline__ int4 read_ids(const Item& it, int t, int l) {
  const uint32_t a =
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) int*)(&g_ids[it.w][t & 7][4 * (l >> 4)]);
  int4 v;
  asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(v) : "v"(a) : "memory");
  return v;
}
// Gather of tile t into K and V slots: instruction u fills rows 4u .. 4u+3,
// lane l taking row 4u + l/16 and logical chunk (l%16) ^ swz(row), so 16
// adjacent lanes read one 256-byte row. Returns the tile's valid-token mask
// (bit r: token r of the tile is in the list and its id is in [0, L)).
// OFF32: the row offsets fit 32 bits (the launch checks), so each address is
// the wave's base plus one 24-bit multiply-add (the load takes the base from
// scalar registers); otherwise they are formed in 64 bits.
template <bool OFF32>
__device__ __forceinline__ uint32_t gather_ids(const Item& it, int t, uint4* kd, uint4* vd,
                                               const int4 ids, int l) {
  const int g = l >> 4, p = l & 15;
  const int idv[4] = {ids.x, ids.y, ids.z, ids.w};
  const int left = it.topk - NT * t;  // rows of the tile inside the list
  bool okv[4];
  bool allok = true;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int r = 4 * u + g;
    const bool ok = r < left && static_cast<unsigned>(idv[u]) < static_cast<unsigned>(it.L);
    okv[u] = ok;
    allok = allok && ok;
    const int row = ok ? idv[u] : 0;
    const int c = p ^ swz(r);
    if constexpr (OFF32) {
      __builtin_assume(static_cast<uint32_t>(row) < (1u << 24));  // row < L < 2^24
      const uint32_t ko = __umul24(static_cast<uint32_t>(row), it.kbytes) + 16u * c;
      const uint32_t vo = __umul24(static_cast<uint32_t>(row), it.vbytes) + 16u * c;
      __builtin_amdgcn_global_load_lds(
          (glb_ptr)(reinterpret_cast<const unsigned char*>(it.kb) + ko), (lds_ptr)(kd + 64 * u),
          16, 0, 0);
      __builtin_amdgcn_global_load_lds(
          (glb_ptr)(reinterpret_cast<const unsigned char*>(it.vb) + vo), (lds_ptr)(vd + 64 * u),
          16, 0, 0);
    } else {
      __builtin_amdgcn_global_load_lds((glb_ptr)(it.kb + static_cast<int64_t>(row) * it.kst + 8 * c),
                                       (lds_ptr)(kd + 64 * u), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((glb_ptr)(it.vb + static_cast<int64_t>(row) * it.vst + 8 * c),
                                       (lds_ptr)(vd + 64 * u), 16, 0, 0);
    }
  }
  // every row valid (all but a list's last tile, unless it has holes)
  if (__ballot(!allok) == 0ull) return 0xFFFFu;
  uint32_t mask = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const uint64_t b = __ballot(okv[u]);
#pragma unroll
    for (int gg = 0; gg < 4; ++gg)
      mask |= static_cast<uint32_t>((b >> (16 * gg)) & 1u) << (4 * u + gg);
  }
  return mask;
}

template <bool OFF32>
__device__ __forceinline__ uint32_t gather(const Item& it, int t, uint4* kd, uint4* vd, int l) {
  return gather_ids<OFF32>(it, t, kd, vd, read_ids(it, t, l), l);
}

struct State {
  bf16x8 qf[4];      // Q^T fragments: head l%16, k 32s + 8(l/16) .. +8
  f32x4 o[8];        // O block dvb: dv 16dvb + l%16, heads 4(l/16) + (0..3)
  float R;           // reference of head l%16 (base 2)
  float lsum;        // partial row sum of head l%16 over this lane's tokens
  uint32_t m0, m1;   // valid masks of tiles t and t+1
  v4s pp;             // bf16 numerators of a pair's even tile (this lane's 4 tokens)
  v4s pv[8];          // its V^T fragments
};

// The fragments of tile t (slot I = t % 2) this lane needs: K fragments
// (row l%16, chunks 4k + l/16) and V^T fragments of the 8 blocks of 16 value
// columns (row 4(l/16) + (l%16)/4, columns 16dvb + 4(l%4) .. +3).
struct Frags {
  uint4 k[4];
  v4s v[8];
};
// With them, the gather ids of tile tid (as read_ids returns them), all in
// one statement that ends with the wait for every LDS read of the wave. The
// reads are written out so that the compiler's load-counter bookkeeping does
// not see them: it cannot tell the ring slots apart from the slot just
// gathered into, and would drain every load in flight (the prefetch of the
// tile two ahead) before the second tile of each loop trip. The slot a read
// names has landed by the load-counter wait that ended the iteration before.
template <int I>
__device__ __forceinline__ int4 read_frags_ids(Frags& f, const Item& it, int tid, int l) {
  const int g = l >> 4, r = l & 15;
  typedef __attribute__((address_space(3))) const unsigned char* lds_byte;
  const uint32_t kt = (uint32_t)(uintptr_t)(lds_byte)(kbuf<I>(it.w));
  const uint32_t vt = (uint32_t)(uintptr_t)(lds_byte)(vbuf<I>(it.w));
  uint32_t ka[4], va[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) ka[k] = kt + 16u * (r * 16 + ((4 * k + g) ^ swz(r)));
  const int vrow = 4 * g + (r >> 2);
  const uint32_t vbase = vt + vrow * 256 + 8 * (r & 1);
#pragma unroll
  for (int dvb = 0; dvb < 8; ++dvb) {
    const int chunk = 2 * dvb + ((r & 3) >> 1);
    va[dvb] = vbase + 16u * (chunk ^ swz(vrow));
  }
  const uint32_t ia = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) int*)(
      &g_ids[it.w][tid & 7][4 * (l >> 4)]);
  int4 ids;
  asm volatile(
      "ds_read_b128 %0, %13\n\t"
      "ds_read_b128 %1, %14\n\t"
      "ds_read_b128 %2, %15\n\t"
      "ds_read_b128 %3, %16\n\t"
      "ds_read_b64_tr_b16 %4, %17\n\t"
      "ds_read_b64_tr_b16 %5, %18\n\t"
      "ds_read_b64_tr_b16 %6, %19\n\t"
      "ds_read_b64_tr_b16 %7, %20\n\t"
      "ds_read_b64_tr_b16 %8, %21\n\t"
      "ds_read_b64_tr_b16 %9, %22\n\t"
      "ds_read_b64_tr_b16 %10, %23\n\t"
      "ds_read_b64_tr_b16 %11, %24\n\t"
      "ds_read_b128 %12, %25\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(f.k[0]), "=&v"(f.k[1]), "=&v"(f.k[2]), "=&v"(f.k[3]), "=&v"(f.v[0]),
        "=&v"(f.v[1]), "=&v"(f.v[2]), "=&v"(f.v[3]), "=&v"(f.v[4]), "=&v"(f.v[5]),
        "=&v"(f.v[6]), "=&v"(f.v[7]), "=&v"(ids)
      : "v"(ka[0]), "v"(ka[1]), "v"(ka[2]), "v"(ka[3]), "v"(va[0]), "v"(va[1]), "v"(va[2]),
        "v"(va[3]), "v"(va[4]), "v"(va[5]), "v"(va[6]), "v"(va[7]), "v"(ia)
      : "memory");
  return ids;
}

// Tile t: S^T, the softmax update, O += P V, from fragments already read.
// The numerators of an even tile wait for the odd tile after it: the pair's
// P V products then run as 16x16x32 MFMAs over the pair's 32 tokens (lane
// group g holding tokens 4g..4g+3 of each tile as its 8 k values, in P and
// in V^T alike), half the instructions of two 16x16x16 rounds.
template <int I>
__device__ __forceinline__ void tile(State& st, const Frags& f, int t,
                                     float scale_log2, int l) {
  const int g = l >> 4;
  // ---- S^T of the tile: lane l gets head l%16, tokens 4g + (0..3); two
  // accumulation chains over the k steps, added at the end
  f32x4 s0 = {0.0f, 0.0f, 0.0f, 0.0f}, s1 = {0.0f, 0.0f, 0.0f, 0.0f};
  s0 = mfma16(as_bf16x8(f.k[0]), st.qf[0], s0);
  s1 = mfma16(as_bf16x8(f.k[1]), st.qf[1], s1);
  s0 = mfma16(as_bf16x8(f.k[2]), st.qf[2], s0);
  s1 = mfma16(as_bf16x8(f.k[3]), st.qf[3], s1);
  // raw scores q.k; the scale (positive, checked by the host) is applied to
  // the tile maximum and inside the numerators' multiply-add
  float sv[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) sv[e] = s0[e] + s1[e];
  if (st.m0 != 0xFFFFu) {  // holes or the list's end: drop the invalid tokens
#pragma unroll
    for (int e = 0; e < 4; ++e) sv[e] = ((st.m0 >> (4 * g + e)) & 1u) ? sv[e] : -INFINITY;
  }
  float tmax = vmax(vmax(sv[0], sv[1]), vmax(sv[2], sv[3]));
  tmax = max_x16_x32(tmax) * scale_log2;
  // ---- reference: set on the first tile, raised when exceeded by far
  const bool up = t == 0 || tmax > st.R + kRaise;
  if (__ballot(up) != 0ull) {
    if constexpr (I % 2 == 1) {
      // the even tile's products first, against the reference they used
#pragma unroll
      for (int dvb = 0; dvb < 8; ++dvb) st.o[dvb] = mfma16k16(st.pp, st.pv[dvb], st.o[dvb]);
      st.pp = v4s{0, 0, 0, 0};
    }
    const float rnew = up ? tmax : st.R;
    const float a = exp2_ratio(st.R, rnew);
    st.lsum *= t == 0 ? 0.0f : a;
    // O rows are heads 4g + e: fetch their factors from the lanes holding them
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float ae = __shfl(a, 4 * g + e, 64);
#pragma unroll
      for (int dvb = 0; dvb < 8; ++dvb) st.o[dvb][e] *= (t == 0 ? 1.0f : ae);
    }
    st.R = rnew;
  }
  const float mneg = st.R == -INFINITY ? 0.0f : -st.R;
  float p[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[e], scale_log2, mneg));
  st.lsum += (p[0] + p[1]) + (p[2] + p[3]);
  const uint2 pp = make_uint2(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]));
  const v4s pa = __builtin_bit_cast(v4s, pp);
  if constexpr (I % 2 == 0) {
    st.pp = pa;
#pragma unroll
    for (int dvb = 0; dvb < 8; ++dvb) st.pv[dvb] = f.v[dvb];
  } else {
    // ---- O += P V over the pair: k values 0..3 from the even tile, 4..7
    // from this one
    const bf16x8 p8 = __builtin_bit_cast(bf16x8, __builtin_shufflevector(st.pp, pa, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
    for (int dvb = 0; dvb < 8; ++dvb) {
      const bf16x8 v8 = __builtin_bit_cast(
          bf16x8, __builtin_shufflevector(st.pv[dvb], f.v[dvb], 0, 1, 2, 3, 4, 5, 6, 7));
      st.o[dvb] = mfma16(p8, v8, st.o[dvb]);
    }
  }
}

// Iteration t (slot t % 2): the K and V fragments of tile t and the gather
// ids of tile t+2, all under one wait; then the gathers of tile t+2 into the
// slot tile t has just left (its data is in registers) and the id load of
// tile t+5; then tile t's products, kept ahead of the wait that ends the
// iteration: at most this iteration's 9 loads (8 gathers, 1 id load) remain,
// so tile t+1 and the ids of tile t+3 have landed.
template <int I, bool OFF32>
__device__ __forceinline__ void iter(State& st, const Item& it, int t,
                                     float scale_log2, int l) {
  Frags f;
  const int4 ids = read_frags_ids<I>(f, it, t + 2, l);
  const uint32_t m2 = gather_ids<OFF32>(it, t + 2, kbuf<I>(it.w), vbuf<I>(it.w), ids, l);
  ids_issue(it, t + 5, l);
  tile<I>(st, f, t, scale_log2, l);
  st.m0 = st.m1;
  st.m1 = m2;
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0x0079);  // vmcnt(9) lgkmcnt(0)
}

}  // namespace d128

using namespace d128;

template <bool OFF32>
__global__ __launch_bounds__(128) void sparse_attn_d128_kernel(
    const uint16_t* __restrict__ q, Str3 qs, const uint16_t* __restrict__ k, Str3 ks,
    const uint16_t* __restrict__ v, Str3 vs, int nq, int L, int Hkv, int G,
    const int32_t* __restrict__ token_idx, int topk, float scale_log2, uint16_t* __restrict__ out,
    Str3 os, float* __restrict__ lse, int64_t nitems, int nsplit, int split_tiles,
    float* __restrict__ part_o, float2* __restrict__ part_rl) {
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), l = threadIdx.x & 63;
  // x = item * nsplit + split; without a split (part_o null) nsplit is 1
  const int64_t x = static_cast<int64_t>(blockIdx.x) * WAVES + w;
  if (x >= nitems * nsplit) return;
  const int64_t item = x / nsplit;
  const int tok0 = static_cast<int>(x % nsplit) * split_tiles * NT;
  // item = (b * nq + qi) * Hkv + gk
  const int gk = static_cast<int>(item % Hkv);
  const int64_t qrow = item / Hkv;
  const int qi = static_cast<int>(qrow % nq), b = static_cast<int>(qrow / nq);
  Item it;
  it.kb = k + b * ks.b + gk * ks.h;
  it.vb = v + b * vs.b + gk * vs.h;
  it.kst = ks.t;
  it.vst = vs.t;
  it.kbytes = static_cast<uint32_t>(2 * ks.t);
  it.vbytes = static_cast<uint32_t>(2 * vs.t);
  it.tix = token_idx + qrow * topk + tok0;
  it.topk = min(topk - tok0, split_tiles * NT);  // >= 1: no split is empty
  it.L = L;
  it.w = w;
  const int ntiles = (it.topk + NT - 1) / NT;
  const int nt2 = (ntiles + 1) & ~1;  // tiles processed: even, the extra one masked

  State st;
  {
    // Q^T fragments: head l%16 (zero past the group), k 32s + 8(l/16)
    const int h = l & 15;
    const uint16_t* qp = q + b * qs.b + qi * qs.t + (gk * G + h) * qs.h + 8 * (l >> 4);
#pragma unroll
    for (int s = 0; s < 4; ++s)
      st.qf[s] = h < G ? as_bf16x8(*reinterpret_cast<const uint4*>(qp + 32 * s))
                       : as_bf16x8(make_uint4(0, 0, 0, 0));
  }
#pragma unroll
  for (int d = 0; d < 8; ++d) st.o[d] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  st.R = -INFINITY;
  st.lsum = 0.0f;
#pragma unroll
  for (int t = 0; t < 5; ++t) ids_issue(it, t, l);
  __builtin_amdgcn_s_waitcnt(0x0070);  // Q and the ids of tiles 0..4
  st.m0 = gather<OFF32>(it, 0, kbuf<0>(w), vbuf<0>(w), l);
  st.m1 = gather<OFF32>(it, 1, kbuf<1>(w), vbuf<1>(w), l);
  __builtin_amdgcn_s_waitcnt(0x0078);  // vmcnt(8): tile 0 has landed
  for (int t = 0; t < nt2; t += 2) {
    iter<0, OFF32>(st, it, t, scale_log2, l);
    iter<1, OFF32>(st, it, t + 1, scale_log2, l);
  }
  __builtin_amdgcn_s_waitcnt(0x0070);  // the loads past the end

  // ---- normalise and store: O rows are heads 4g + e; their row sums and
  // references sit in the lanes whose column is that head
  const float ltot = sum_x16_x32(st.lsum);
  const int g = l >> 4;
  if (part_o != nullptr) {
    // this split's unnormalised O (rows = heads), reference and row sum
    float* po = part_o + x * (static_cast<int64_t>(G) * D);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int h = 4 * g + e;
      if (h < G) {
#pragma unroll
        for (int dvb = 0; dvb < 8; ++dvb) po[h * D + 16 * dvb + (l & 15)] = st.o[dvb][e];
      }
    }
    if (l < G) part_rl[x * G + l] = make_float2(st.R, ltot);
    return;
  }
  uint16_t* orow = out + b * os.b + qi * os.t + gk * G * os.h;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int h = 4 * g + e;
    const float lh = __shfl(ltot, h, 64);
    const float inv = lh > 0.0f ? 1.0f / lh : 0.0f;
    if (h < G) {
#pragma unroll
      for (int dvb = 0; dvb < 8; ++dvb)
        orow[h * os.h + 16 * dvb + (l & 15)] = f32_to_bf16(st.o[dvb][e] * inv);
    }
  }
  if (lse != nullptr && l < 16 && l < G)
    lse[qrow * (static_cast<int64_t>(G) * Hkv) + gk * G + l] =
        ltot > 0.0f ? (st.R + log2f(ltot)) * 0.69314718055994530942f : -INFINITY;
}

// The splits of one item, rescaled to their largest reference and summed:
// workgroup (item, head pair), thread = one output column of one head.
__global__ __launch_bounds__(256) void attn_d128_combine_kernel(
    const float* __restrict__ part_o, const float2* __restrict__ part_rl, int nsplit, int nq,
    int Hkv, int G, uint16_t* __restrict__ out, Str3 os, float* __restrict__ lse) {
  const int64_t item = blockIdx.x;
  const int h = 2 * blockIdx.y + (threadIdx.x >> 7);
  const int c = threadIdx.x & (D - 1);
  if (h >= G) return;
  const float2* rl = part_rl + item * nsplit * G + h;
  const float* po = part_o + (item * nsplit * G + h) * D + c;
  // the splits in groups of 8 whose loads are all issued before they are used
  float M = -INFINITY;
  for (int s0 = 0; s0 < nsplit; s0 += 8) {
    float2 a[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      a[u] = s0 + u < nsplit ? rl[(s0 + u) * G] : make_float2(-INFINITY, 0.0f);
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (a[u].y > 0.0f) M = fmaxf(M, a[u].x);
  }
  float lt = 0.0f, acc = 0.0f;
  for (int s0 = 0; s0 < nsplit; s0 += 8) {
    float2 a[8];
    float o[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const bool ok = s0 + u < nsplit;
      a[u] = ok ? rl[(s0 + u) * G] : make_float2(-INFINITY, 0.0f);
      o[u] = ok ? po[static_cast<int64_t>(s0 + u) * G * D] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (a[u].y > 0.0f) {
        const float f = exp2_ratio(a[u].x, M);
        lt += a[u].y * f;
        acc += o[u] * f;
      }
    }
  }
  const int gk = static_cast<int>(item % Hkv);
  const int64_t qrow = item / Hkv;
  const int qi = static_cast<int>(qrow % nq), b = static_cast<int>(qrow / nq);
  out[b * os.b + qi * os.t + (gk * G + h) * os.h + c] = f32_to_bf16(lt > 0.0f ? acc / lt : 0.0f);
  if (lse != nullptr && c == 0)
    lse[qrow * (static_cast<int64_t>(G) * Hkv) + gk * G + h] =
        lt > 0.0f ? (M + log2f(lt)) * 0.69314718055994530942f : -INFINITY;
}

// Splits of each token list: enough waves to occupy the chip, at least
// kMinSplitTiles tiles each, none empty.
static int d128_splits(int64_t nitems, int topk, int* split_tiles) {
  const int ntiles = (topk + NT - 1) / NT;
  int64_t s = std::min<int64_t>((kSplitWaves + nitems - 1) / nitems, ntiles / kMinSplitTiles);
  s = std::max<int64_t>(s, 1);
  const int tps = static_cast<int>((ntiles + s - 1) / s);
  *split_tiles = tps;
  return (ntiles + tps - 1) / tps;
}

size_t attn_d128_workspace(int batch, int nq, int Hkv, int G, int topk) {
  const int64_t nitems = static_cast<int64_t>(batch) * nq * Hkv;
  int tps;
  const int ns = d128_splits(nitems, topk, &tps);
  if (ns <= 1) return 0;
  const size_t n = static_cast<size_t>(nitems) * ns * G;
  return align256(n * D * 4) + align256(n * 8);
}

hipError_t launch_attn_d128(const uint16_t* q, Str3 qs, const uint16_t* k, Str3 ks,
                            const uint16_t* v, Str3 vs, int batch, int nq, int L, int Hkv, int G,
                            const int32_t* token_idx, int topk, float scale, uint16_t* out,
                            Str3 os, float* lse, void* ws, hipStream_t s) {
  const int64_t nitems = static_cast<int64_t>(batch) * nq * Hkv;
  int tps;
  int ns = d128_splits(nitems, topk, &tps);
  if (ws == nullptr || ns <= 1) {  // one wave per item
    ns = 1;
    tps = (topk + NT - 1) / NT;
  }
  float* part_o = nullptr;
  float2* part_rl = nullptr;
  if (ns > 1) {
    const size_t n = static_cast<size_t>(nitems) * ns * G;
    part_o = static_cast<float*>(ws);
    part_rl = reinterpret_cast<float2*>(static_cast<char*>(ws) + align256(n * D * 4));
  }
  const int64_t waves = nitems * ns;
  const unsigned blocks = static_cast<unsigned>((waves + WAVES - 1) / WAVES);
  // 32-bit row offsets when every row of the cache lies within 4 GB of its
  // base and the byte strides fit the 24-bit multiply
  const int64_t span = (static_cast<int64_t>(L) - 1) * std::max(ks.t, vs.t) * 2 + 2 * D;
  const bool off32 = span < (int64_t{1} << 32) && L < (1 << 24) && 2 * ks.t < (1 << 24) &&
                     2 * vs.t < (1 << 24);
  if (off32)
    hipLaunchKernelGGL(sparse_attn_d128_kernel<true>, dim3(blocks), dim3(64 * WAVES), 0, s, q, qs,
                       k, ks, v, vs, nq, L, Hkv, G, token_idx, topk,
                       scale * 1.44269504088896340736f, out, os, lse, nitems, ns, tps, part_o,
                       part_rl);
  else
    hipLaunchKernelGGL(sparse_attn_d128_kernel<false>, dim3(blocks), dim3(64 * WAVES), 0, s, q,
                       qs, k, ks, v, vs, nq, L, Hkv, G, token_idx, topk,
                       scale * 1.44269504088896340736f, out, os, lse, nitems, ns, tps, part_o,
                       part_rl);
  if (ns > 1)
    hipLaunchKernelGGL(attn_d128_combine_kernel,
                       dim3(static_cast<unsigned>(nitems), static_cast<unsigned>((G + 1) / 2)),
                       dim3(256), 0, s, part_o, part_rl, ns, nq, Hkv, G, out, os, lse);
  return hipGetLastError();
}

}  // namespace hisa
