// Token level: score every token of the kept blocks and keep the top k
// (HISA explainer 1.2.2; HISA news article, "fine token selection"), plus
// the flat comparison indexer that scores every causal token (HISA
// explainer 1.1 item 1).
//
// Hierarchical path, block-major: each query keeps m different blocks, so a
// query-major product degenerates to a gather-bound matrix-vector product.
// Instead the (query, slot) pairs are bucketed by key block (counting sort),
// and each workgroup multiplies one key block (B tokens x d) by up to 64
// gathered query rows on the bf16 matrix cores (fp32 accumulation, exact for
// integer-valued indexer data). Scores land in a per-query candidate buffer
// [query][slot][B] whose position order is ascending token id, and one
// workgroup per query then selects the top k from it.
#include <algorithm>
#include <mutex>

#include "common.hpp"
#include "internal.h"
#include "select.hpp"

namespace hisa {

constexpr int kTQ = 64;  // pairs per scoring tile
// keys per thread and per workgroup of the bucket-count scan
constexpr int kScanPer = 16, kScanChunk = 256 * kScanPer;

static_assert(kTQ == kPairTile, "token scoring tiles are pair-bucket tiles");

PairBuckets carve_pair_buckets(void* ws, int batch, int nq, int m, int nblk, size_t* bytes) {
  const size_t nkeys = static_cast<size_t>(batch) * nblk;
  const size_t npairs = static_cast<size_t>(batch) * nq * m;
  const size_t max_tiles = (npairs + kTQ - 1) / kTQ + nkeys;
  char* p = static_cast<char*>(ws);
  size_t off = 0;
  PairBuckets w;
  auto take = [&](size_t n) { char* r = p ? p + off : nullptr; off += align256(n); return r; };
  w.cnt = reinterpret_cast<uint32_t*>(take(nkeys * 4));
  w.cursor = reinterpret_cast<uint32_t*>(take(nkeys * 4));
  w.offs = reinterpret_cast<uint32_t*>(take(nkeys * 4));
  w.tile_off = reinterpret_cast<uint32_t*>(take(nkeys * 4));
  w.total = reinterpret_cast<uint32_t*>(take(16));
  w.part = reinterpret_cast<uint32_t*>(take(2 * 4 * ((nkeys + kScanChunk - 1) / kScanChunk)));
  w.pairs = reinterpret_cast<uint32_t*>(take(npairs * 4));
  w.tiles = reinterpret_cast<uint32_t*>(take(max_tiles * 4));
  if (bytes) *bytes = off;
  return w;
}

struct TokWs : PairBuckets {
  float* scores;        // [batch*nq*m*B]
};

// The row top-k loads whole waves of 64-score rows from a query's first row,
// up to 256 rows (W * RW), whether or not the query has that many: rows past
// its own are masked, and the buffer ends with this much slack so that the
// last query's loads stay inside it.
constexpr size_t kScoreTailPad = static_cast<size_t>(256) * 64 * 4;

static TokWs carve(void* ws, int batch, int nq, int L, int B, int m, size_t* bytes) {
  const int nblk = (L + B - 1) / B;
  const size_t npairs = static_cast<size_t>(batch) * nq * m;
  size_t off = 0;
  TokWs w;
  static_cast<PairBuckets&>(w) = carve_pair_buckets(ws, batch, nq, m, nblk, &off);
  w.scores = ws ? reinterpret_cast<float*>(static_cast<char*>(ws) + off) : nullptr;
  off += align256(npairs * B * 4 + kScoreTailPad);
  if (bytes) *bytes = off;
  return w;
}

size_t token_select_workspace(int batch, int nq, int L, int B, int m, int /*k*/) {
  size_t bytes = 0;
  carve(nullptr, batch, nq, L, B, m, &bytes);
  return bytes;
}

// ------------------------------------------------------------ fixed scratch
// The scratch of the allocation-free token selection: one array in device
// memory per GPU, held from the library's load on that GPU until the process
// ends. In host code `scratch` only names the symbol; its device address on
// each GPU comes from hipGetSymbolAddress and is the only form passed on.
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

hipError_t noalloc_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    // once per device, with that device current
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

// ------------------------------------------------------------ pair buckets
__global__ void zero_u32_kernel(uint32_t* __restrict__ p, size_t n) {
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    p[i] = 0u;
}

// Bucket counts with per-workgroup aggregation: one workgroup takes `qpw`
// consecutive queries of one sequence, counts their blocks in an LDS
// histogram, then adds each non-empty bin to the global count with one
// atomic. Block 0 and the local blocks are shared by thousands of queries, so
// direct global atomics would serialise on a few addresses.
constexpr int kHistMax = 8192;  // largest block count with LDS histograms (64 KB)

__global__ __launch_bounds__(256) void count_pairs_kernel(const int32_t* __restrict__ block_idx,
                                                          int nq, int m, int nblk, int qpw,
                                                          uint32_t* __restrict__ cnt) {
  extern __shared__ uint32_t hist[];
  const int b = blockIdx.y;
  const int q0 = blockIdx.x * qpw, q1 = min(nq, q0 + qpw);
  for (int c = threadIdx.x; c < nblk; c += 256) hist[c] = 0u;
  __syncthreads();
  const int32_t* bi = block_idx + (static_cast<int64_t>(b) * nq + q0) * m;
  const int n = (q1 - q0) * m;
  for (int i = threadIdx.x; i < n; i += 256) {
    const int c = bi[i];
    if (c >= 0 && c < nblk) atomicAdd(&hist[c], 1u);
  }
  __syncthreads();
  uint32_t* cb = cnt + static_cast<int64_t>(b) * nblk;
  for (int c = threadIdx.x; c < nblk; c += 256)
    if (hist[c] != 0u) atomicAdd(&cb[c], hist[c]);
}

// Exclusive scans of the bucket counts (pair offsets and tile offsets) in
// key order, in chunks of 4096 keys: thread t of a chunk's workgroup holds
// keys 16t .. 16t+15, loaded as four 16-byte vectors. With more than one
// chunk, a first kernel writes each chunk's two sums and the scan kernel adds
// those of the chunks before its own.
__device__ __forceinline__ uint32_t tiles_of(uint32_t c) { return (c + kTQ - 1) / kTQ; }

__device__ __forceinline__ void load_counts(const uint32_t* __restrict__ cnt, int nkeys, int k0,
                                            uint32_t (&c)[kScanPer]) {
  if (k0 + kScanPer <= nkeys) {
#pragma unroll
    for (int j = 0; j < kScanPer / 4; ++j) {
      const uint4 u = *reinterpret_cast<const uint4*>(cnt + k0 + 4 * j);
      c[4 * j + 0] = u.x;
      c[4 * j + 1] = u.y;
      c[4 * j + 2] = u.z;
      c[4 * j + 3] = u.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kScanPer; ++j) c[j] = k0 + j < nkeys ? cnt[k0 + j] : 0u;
  }
}

__global__ __launch_bounds__(256) void bucket_partials_kernel(const uint32_t* __restrict__ cnt,
                                                              int nkeys,
                                                              uint32_t* __restrict__ part) {
  __shared__ uint32_t red[4];
  uint32_t c[kScanPer];
  load_counts(cnt, nkeys, blockIdx.x * kScanChunk + threadIdx.x * kScanPer, c);
  uint32_t sp = 0, st = 0;
#pragma unroll
  for (int j = 0; j < kScanPer; ++j) {
    sp += c[j];
    st += tiles_of(c[j]);
  }
  sp = block_sum<256>(sp, red);
  st = block_sum<256>(st, red);
  if (threadIdx.x == 0) {
    part[2 * blockIdx.x] = sp;
    part[2 * blockIdx.x + 1] = st;
  }
}

// part == nullptr: one chunk only
__global__ __launch_bounds__(256) void scan_buckets_kernel(const uint32_t* __restrict__ cnt,
                                                           int nkeys,
                                                           const uint32_t* __restrict__ part,
                                                           int nchunks, uint32_t* __restrict__ offs,
                                                           uint32_t* __restrict__ tile_off,
                                                           uint32_t* __restrict__ total) {
  __shared__ uint32_t red[4];
  const int k0 = blockIdx.x * kScanChunk + threadIdx.x * kScanPer;
  uint32_t c[kScanPer];
  load_counts(cnt, nkeys, k0, c);
  uint32_t bp = 0, bt = 0, ap = 0, at = 0;  // chunks before this one; all chunks
  if (part) {
    for (int i = threadIdx.x; i < nchunks; i += 256) {
      const uint32_t p = part[2 * i], t = part[2 * i + 1];
      ap += p;
      at += t;
      bp += i < static_cast<int>(blockIdx.x) ? p : 0u;
      bt += i < static_cast<int>(blockIdx.x) ? t : 0u;
    }
    bp = block_sum<256>(bp, red);
    bt = block_sum<256>(bt, red);
    ap = block_sum<256>(ap, red);
    at = block_sum<256>(at, red);
  }
  uint32_t sp = 0, st = 0;
#pragma unroll
  for (int j = 0; j < kScanPer; ++j) {
    sp += c[j];
    st += tiles_of(c[j]);
  }
  uint32_t tp, tt;
  uint32_t ep = bp + block_excl_scan<256>(sp, tp, red);
  uint32_t et = bt + block_excl_scan<256>(st, tt, red);
  uint32_t o[kScanPer], to[kScanPer];
#pragma unroll
  for (int j = 0; j < kScanPer; ++j) {
    o[j] = ep;
    to[j] = et;
    ep += c[j];
    et += tiles_of(c[j]);
  }
  if (k0 + kScanPer <= nkeys) {
#pragma unroll
    for (int j = 0; j < kScanPer / 4; ++j) {
      *reinterpret_cast<uint4*>(offs + k0 + 4 * j) =
          make_uint4(o[4 * j], o[4 * j + 1], o[4 * j + 2], o[4 * j + 3]);
      *reinterpret_cast<uint4*>(tile_off + k0 + 4 * j) =
          make_uint4(to[4 * j], to[4 * j + 1], to[4 * j + 2], to[4 * j + 3]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < kScanPer; ++j)
      if (k0 + j < nkeys) {
        offs[k0 + j] = o[j];
        tile_off[k0 + j] = to[j];
      }
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    total[0] = part ? ap : tp;
    total[1] = part ? at : tt;
  }
}

// Scatter with the same aggregation: each workgroup reserves one contiguous
// range per non-empty bucket, then ranks its own entries inside it.
__global__ __launch_bounds__(256) void scatter_pairs_kernel(
    const int32_t* __restrict__ block_idx, int nq, int m, int nblk, int qpw,
    const uint32_t* __restrict__ offs, uint32_t* __restrict__ cursor,
    uint32_t* __restrict__ pairs) {
  extern __shared__ uint32_t hist[];  // [0, nblk): counts then bases; [nblk, 2nblk): ranks
  uint32_t* rank = hist + nblk;
  const int b = blockIdx.y;
  const int q0 = blockIdx.x * qpw, q1 = min(nq, q0 + qpw);
  for (int c = threadIdx.x; c < nblk; c += 256) {
    hist[c] = 0u;
    rank[c] = 0u;
  }
  __syncthreads();
  const int64_t e0 = (static_cast<int64_t>(b) * nq + q0) * m;
  const int32_t* bi = block_idx + e0;
  const int n = (q1 - q0) * m;
  for (int i = threadIdx.x; i < n; i += 256) {
    const int c = bi[i];
    if (c >= 0 && c < nblk) atomicAdd(&hist[c], 1u);
  }
  __syncthreads();
  const int64_t kb = static_cast<int64_t>(b) * nblk;
  for (int c = threadIdx.x; c < nblk; c += 256) {
    const uint32_t h = hist[c];
    if (h != 0u) hist[c] = offs[kb + c] + atomicAdd(&cursor[kb + c], h);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += 256) {
    const int c = bi[i];
    if (c >= 0 && c < nblk) pairs[hist[c] + atomicAdd(&rank[c], 1u)] = static_cast<uint32_t>(e0 + i);
  }
}

// Fallback for very many blocks per sequence: one global atomic per entry.
__global__ void count_pairs_direct_kernel(const int32_t* __restrict__ block_idx, int nq, int m,
                                          int nblk, size_t npairs, uint32_t* __restrict__ cnt) {
  const size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x;
  if (i >= npairs) return;
  const int c = block_idx[i];
  if (c < 0 || c >= nblk) return;
  const size_t b = i / (static_cast<size_t>(nq) * m);
  atomicAdd(&cnt[b * nblk + c], 1u);
}
__global__ void scatter_pairs_direct_kernel(const int32_t* __restrict__ block_idx, int nq, int m,
                                            int nblk, size_t npairs,
                                            const uint32_t* __restrict__ offs,
                                            uint32_t* __restrict__ cursor,
                                            uint32_t* __restrict__ pairs) {
  const size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x;
  if (i >= npairs) return;
  const int c = block_idx[i];
  if (c < 0 || c >= nblk) return;
  const size_t key = (i / (static_cast<size_t>(nq) * m)) * nblk + c;
  const uint32_t pos = offs[key] + atomicAdd(&cursor[key], 1u);
  pairs[pos] = static_cast<uint32_t>(i);
}

__global__ void tile_table_kernel(const uint32_t* __restrict__ cnt,
                                  const uint32_t* __restrict__ tile_off, int nkeys,
                                  uint32_t* __restrict__ tiles) {
  const int key = blockIdx.x * blockDim.x + threadIdx.x;
  if (key >= nkeys) return;
  const uint32_t nt = (cnt[key] + kTQ - 1) / kTQ;
  for (uint32_t t = 0; t < nt; ++t) tiles[tile_off[key] + t] = static_cast<uint32_t>(key);
}

// Buckets of (query, slot) entries by (sequence, block), then the tile table:
// entry e = (b*nq + q)*m + slot of block_idx goes to bucket b*nblk + block;
// bucket k holds pairs[offs[k] .. offs[k] + cnt[k]) in no particular order,
// split into tiles of kPairTile entries numbered from tile_off[k], and
// tiles[i] names the bucket of tile i (total[0] entries, total[1] tiles).
hipError_t launch_pair_buckets(const int32_t* block_idx, int batch, int nq, int m, int nblk,
                               const PairBuckets& w, hipStream_t s) {
  const int nkeys = batch * nblk;
  const size_t npairs = static_cast<size_t>(batch) * nq * m;
  // cnt and cursor are adjacent: clear both with one fill kernel
  const size_t zero_n = (reinterpret_cast<char*>(w.offs) - reinterpret_cast<char*>(w.cnt)) / 4;
  hipLaunchKernelGGL(zero_u32_kernel, dim3(std::min<size_t>((zero_n + 255) / 256, 4096)),
                     dim3(256), 0, s, w.cnt, zero_n);
  const unsigned pg = static_cast<unsigned>((npairs + 255) / 256);
  const bool lds_hist = nblk <= kHistMax;
  const int qpw = std::max(1, 4096 / m);
  const dim3 hg((nq + qpw - 1) / qpw, batch);
  if (lds_hist)
    hipLaunchKernelGGL(count_pairs_kernel, hg, dim3(256), nblk * 4, s, block_idx, nq, m, nblk,
                       qpw, w.cnt);
  else
    hipLaunchKernelGGL(count_pairs_direct_kernel, dim3(pg), dim3(256), 0, s, block_idx, nq, m,
                       nblk, npairs, w.cnt);
  const int nchunks = (nkeys + kScanChunk - 1) / kScanChunk;
  if (nchunks > 1)
    hipLaunchKernelGGL(bucket_partials_kernel, dim3(nchunks), dim3(256), 0, s, w.cnt, nkeys,
                       w.part);
  hipLaunchKernelGGL(scan_buckets_kernel, dim3(nchunks), dim3(256), 0, s, w.cnt, nkeys,
                     nchunks > 1 ? w.part : nullptr, nchunks, w.offs, w.tile_off, w.total);
  if (lds_hist)
    hipLaunchKernelGGL(scatter_pairs_kernel, hg, dim3(256), nblk * 8, s, block_idx, nq, m, nblk,
                       qpw, w.offs, w.cursor, w.pairs);
  else
    hipLaunchKernelGGL(scatter_pairs_direct_kernel, dim3(pg), dim3(256), 0, s, block_idx, nq, m,
                       nblk, npairs, w.offs, w.cursor, w.pairs);
  hipLaunchKernelGGL(tile_table_kernel, dim3((nkeys + 255) / 256), dim3(256), 0, s, w.cnt,
                     w.tile_off, nkeys, w.tiles);
  return hipGetLastError();
}

// ------------------------------------------------------------ scoring
// S^T[token, pair] = K_blk[token, :] . Q[pair, :]. Wave w owns tokens
// [w*BS/4, (w+1)*BS/4) of the key block (A operand, straight from global),
// all 64 pairs of the tile are the B operand: their query rows are gathered
// once per workgroup into LDS (rows padded by 16 bytes), which every wave
// reads (each wave gathering them itself read them four times: 64K token
// select 2.25 -> 2.07 ms). The
// accumulator lane layout (column = pair, 4 consecutive tokens) is stored
// as one 16-byte write per pair.
template <int D, int BS>
__global__ __launch_bounds__(256) void token_score_kernel(
    const uint16_t* __restrict__ qidx, int64_t qsb, int64_t qst, const uint16_t* __restrict__ kidx,
    int64_t ksb, int64_t kst, int L, int nq, int m, int nblk, const uint32_t* __restrict__ tiles,
    const uint32_t* __restrict__ total, const uint32_t* __restrict__ tile_off,
    const uint32_t* __restrict__ offs, const uint32_t* __restrict__ cnt,
    const uint32_t* __restrict__ pairs, float* __restrict__ scores) {
  constexpr int KS = D / 32;
  constexpr int MT = BS / 64;  // 16-token tiles per wave
  constexpr int TPW = BS / 4;  // first token of wave w: w * TPW
  const uint32_t tile = blockIdx.x;
  if (tile >= total[1]) return;
  const uint32_t key = tiles[tile];
  const uint32_t sub = tile - tile_off[key];
  const uint32_t p0 = offs[key] + sub * kTQ;
  const uint32_t np = min(static_cast<uint32_t>(kTQ), cnt[key] - sub * kTQ);
  const int b = key / nblk;
  const int c = key % nblk;
  const int wave = threadIdx.x / kWave, lane = lane_id();
  const int g = lane / 16, r16 = lane % 16;
  // the tile's query rows, gathered once into LDS (every wave needs all of them)
  constexpr int QRS = 2 * D + 16;  // padded row stride (bytes)
  __shared__ __align__(16) unsigned char qs_lds[kTQ * QRS];
  for (int x = threadIdx.x; x < kTQ * (D / 8); x += 256) {
    const int pr = x / (D / 8), ch = x % (D / 8);
    const uint32_t pl = min(static_cast<uint32_t>(pr), np - 1);
    const uint32_t qrow = pairs[p0 + pl] / m;
    const int qq = qrow % nq;
    *reinterpret_cast<uint4*>(qs_lds + pr * QRS + 16 * ch) = *reinterpret_cast<const uint4*>(
        qidx + b * qsb + static_cast<int64_t>(qq) * qst + 8 * ch);
  }

  bf16x8 a[MT][KS];
  const int tok0 = c * BS + wave * TPW;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int j = min(tok0 + mt * 16 + r16, L - 1);
    const uint16_t* kr = kidx + b * ksb + static_cast<int64_t>(j) * kst + 8 * g;
#pragma unroll
    for (int s = 0; s < KS; ++s) a[mt][s] = as_bf16x8(*reinterpret_cast<const uint4*>(kr + 32 * s));
  }
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    if (nt * 16 >= static_cast<int>(np)) break;
    const uint32_t pl = min(static_cast<uint32_t>(nt * 16 + r16), np - 1);
    const uint32_t pid = pairs[p0 + pl];
    bf16x8 bq[KS];
    if (nt == 0) __syncthreads();  // query rows staged
#pragma unroll
    for (int s = 0; s < KS; ++s)
      bq[s] = as_bf16x8(*reinterpret_cast<const uint4*>(qs_lds + (nt * 16 + r16) * QRS + 64 * s +
                                                         16 * g));
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < KS; ++s) acc = mfma16(a[mt][s], bq[s], acc);
      if (nt * 16 + r16 < static_cast<int>(np)) {
        const int tk = wave * TPW + mt * 16 + 4 * g;
        *reinterpret_cast<f32x4*>(scores + static_cast<int64_t>(pid) * BS + tk) = acc;
      }
    }
  }
}

// The direct form on the VALU: one query against one key block, with no
// other query to share the block's rows (a matrix-core tile would use one
// of its 16 columns). Wave gw scores tokens 32(gw mod BS/32) .. +31 of pair
// gw / (BS/32). A key row is read by D/8 adjacent lanes, 16 bytes each, so
// every load instruction reads whole 128-byte lines (64 / (D/8) rows); each
// lane takes the dot product of its 8 key elements with the matching 8
// query elements (fp32 multiply-adds in element order) and the row's lanes
// are summed with in-row lane moves. All loads are issued before any
// arithmetic. Integer-valued keys and queries give exact scores in any order.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __uint_as_float(static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(__float_as_uint(x)), CTRL, 0xf, 0xf, false)));
}
// Sum over each group of LPR adjacent lanes (8 or 16), in every lane of it.
template <int LPR>
__device__ __forceinline__ float row_lanes_sum(float v) {
  v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(v);  // row_half_mirror: lane i <-> 7 - i of each 8
  if constexpr (LPR == 16) v += dpp_f<0x140>(v);  // row_mirror: lane i <-> 15 - i
  return v;
}

template <int D, int BS>
__global__ __launch_bounds__(256) void token_score_direct_kernel(
    const uint16_t* __restrict__ qidx, int64_t qsb, int64_t qst, const uint16_t* __restrict__ kidx,
    int64_t ksb, int64_t kst, int L, int nq, int m, int nblk,
    const int32_t* __restrict__ block_idx, float* __restrict__ scores, uint32_t npairs) {
  constexpr int LPR = D / 8;     // lanes per key row
  constexpr int RPI = 64 / LPR;  // rows per load instruction
  constexpr int TPW = 32;        // tokens per wave
  constexpr int WPP = BS / TPW;  // waves per pair
  constexpr int NI = TPW / RPI;  // load instructions per wave
  static_assert(BS % TPW == 0 && (LPR == 8 || LPR == 16), "shape");
  const int wave = threadIdx.x / kWave, l = lane_id();
  const uint32_t gw = blockIdx.x * 4u + static_cast<uint32_t>(wave);
  const uint32_t pair = gw / WPP;
  if (pair >= npairs) return;
  const int c = block_idx[pair];
  if (c < 0 || c >= nblk) return;  // empty slot: never a candidate
  const int b = static_cast<int>(pair / (static_cast<uint32_t>(nq) * m));
  const int qq = static_cast<int>((pair / m) % nq);
  const int p = l % LPR, r = l / LPR;
  const int w0 = static_cast<int>(gw % WPP) * TPW;  // first token of this wave in the block
  const int tok0 = c * BS + w0;
  const uint16_t* kb = kidx + b * ksb + 8 * p;
  uint4 kv[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int j = min(tok0 + i * RPI + r, L - 1);
    kv[i] = *reinterpret_cast<const uint4*>(kb + static_cast<int64_t>(j) * kst);
  }
  const uint4 qv = *reinterpret_cast<const uint4*>(qidx + b * qsb + static_cast<int64_t>(qq) * qst +
                                                   8 * p);
  const float qf[8] = {bf16_lo(qv.x), bf16_hi(qv.x), bf16_lo(qv.y), bf16_hi(qv.y),
                       bf16_lo(qv.z), bf16_hi(qv.z), bf16_lo(qv.w), bf16_hi(qv.w)};
  float* out = scores + static_cast<int64_t>(pair) * BS + w0;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const uint32_t e[4] = {kv[i].x, kv[i].y, kv[i].z, kv[i].w};
    float sv = 0.0f;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      sv = __builtin_fmaf(bf16_lo(e[h]), qf[2 * h], sv);
      sv = __builtin_fmaf(bf16_hi(e[h]), qf[2 * h + 1], sv);
    }
    sv = row_lanes_sum<LPR>(sv);
    if (p == 0) out[i * RPI + r] = sv;
  }
}

// ------------------------------------------------------------ selection
// One workgroup (256 threads) per query; thread t owns candidate positions
// t*ITEMS .. t*ITEMS+ITEMS-1 of the query's [m][B] buffer (slot-major, so
// position order is ascending token id). Tokens after the query and empty
// slots are not candidates.
template <int ITEMS>
__global__ __launch_bounds__(256) void token_topk_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ block_idx,
    const int32_t* __restrict__ q_pos, int m, int B, int k, int L, int32_t* __restrict__ token_idx,
    float* __restrict__ token_scores) {
  constexpr int NT = 256, NB = 2048;
  __shared__ SelectLds<NT, NB> sh;
  __shared__ int blk[1024];
  const int64_t qi = blockIdx.x;
  const int t = min(max(q_pos[qi], 0), L - 1);
  const int nblk = (L + B - 1) / B;
  for (int i = threadIdx.x; i < m; i += NT) {
    const int c = block_idx[qi * m + i];
    blk[i] = c < nblk ? c : -1;
  }
  __syncthreads();
  const float* row = scores + qi * m * B;
  const int n_all = m * B;
  float vals[ITEMS];
  bool ok[ITEMS];
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const int p = threadIdx.x * ITEMS + i;
    ok[i] = false;
    vals[i] = 0.0f;
    if (p < n_all) {
      const int c = blk[p / B];
      const int j = c * B + p % B;
      if (c >= 0 && j <= t) {
        ok[i] = true;
        vals[i] = row[p];
      }
    }
  }
  auto get = [&](int, int i, float& v) -> bool {
    v = vals[i];
    return ok[i];
  };
  const Threshold th = select_threshold<NT, ITEMS, NB>(get, 1, k, sh);
  uint32_t kept = 0, ties = 0;
  int32_t* oi = token_idx + qi * k;
  float* os = token_scores ? token_scores + qi * k : nullptr;
  select_compact<NT, ITEMS, NB>(get, 0, th, kept, ties, sh, [&](uint32_t pos, int i, float v) {
    const int p = threadIdx.x * ITEMS + i;
    oi[pos] = blk[p / B] * B + p % B;
    if (os) os[pos] = v;
  });
  for (int i = kept + threadIdx.x; i < k; i += NT) {
    oi[i] = -1;
    if (os) os[i] = __uint_as_float(0x7fc00000u);
  }
}

// The same selection with the candidates laid out by rows: one workgroup of
// W waves per query, wave w holding rows RW*w .. RW*w+RW-1, lane l position
// 64r + l of row r. Each row is one slot's 64 consecutive tokens (B is a
// multiple of 64), so the slot's block id is uniform per row and the loads
// are coalesced. Candidates that are not valid (empty slot, token after the
// query) are held as the quiet NaN 0x7fc00000, which no comparison keeps.
// Scores of valid candidates are finite (products of finite bf16 rows).
//
// The threshold search is specialised for candidates held in registers:
//   1. min and max of the candidates (the count comes from the row bounds);
//   2. a histogram of kRowBins linear bins over [min, max] (LDS atomics) and
//      the bin beta holding the K-th largest value, with the count above it;
//   3. if beta holds at most kRowList candidates they are copied to LDS and
//      every wave ranks them (each against all of them) to find the
//      (K - above)-th largest exactly; otherwise the range shrinks to the
//      bin's own min and max and step 2 repeats (at most kRowLevels times),
//      an exact bisection on order-preserving keys finishing a search that
//      is still open.
// The bins are a monotone function of the value, so every candidate of a
// higher bin is larger than every candidate of bin beta, and the ranks
// inside the bin decide the threshold T and the number of candidates equal
// to T that are kept. The compaction ranks each row with ballots and takes
// the waves' offsets from one exchange of their counts.
constexpr int kRowBins = 2048;
constexpr int kRowList = 64;
constexpr int kRowLevels = 3;

template <int W>
struct RowSelLds {
  uint32_t hist[kRowBins];
  float wmn[W], wmx[W];
  uint32_t wn[W];
  uint32_t part[W];
  uint32_t wcnt[2][W];
  float list[W][kRowList];
  uint32_t nlist[W];
  int beta;
  uint32_t above, hbeta;
};

struct RowThreshold {
  float T;    // values > T are kept
  int need;   // plus the first `need` values == T
  bool all;   // every value == T is kept: keep exactly the values >= T
};

// min / max that pass over the non-candidates: with a quiet NaN operand the
// instructions return the other operand. Written out because the library
// forms first quieten each operand, an instruction per candidate.
__device__ __forceinline__ float min_skip_nan(float a, float b) {
  float r;
  asm("v_min_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float max_skip_nan(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
// float -> int32 rounding towards zero, saturating, NaN -> 0 (the
// instruction's defined behaviour, which the C++ conversion leaves undefined)
__device__ __forceinline__ int cvt_i32_nan0(float x) {
  int r;
  asm("v_cvt_i32_f32 %0, %1" : "=v"(r) : "v"(x));
  return r;
}
// An opaque copy of a pass's parameter: each pass compares the candidates
// against its own copy, so that no pass reuses the compares of an earlier
// one, which would keep them as lane masks, two scalar registers per row.
__device__ __forceinline__ float fresh(float x) {
  asm volatile("" : "+v"(x));
  return x;
}
__device__ __forceinline__ int fresh(int x) {
  asm volatile("" : "+v"(x));
  return x;
}
// Lanes of the wave for which p holds. The count is taken in an ordered
// (volatile) statement so that each row's lane mask dies at once: left to
// the compiler, the compares of all rows are issued ahead of the counts and
// their masks, two scalar registers each, spill.
__device__ __forceinline__ uint32_t row_count(bool p) {
  const uint64_t m = __ballot(p);
  uint32_t c;
  asm volatile("s_bcnt1_i32_b64 %0, %1" : "=s"(c) : "s"(m));
  return c;
}

// Sum over the workgroup of a wave-uniform count (two barriers).
template <int W>
__device__ __forceinline__ uint32_t rows_block_sum(uint32_t c, RowSelLds<W>& sh, int wv, int l) {
  if (l == 0) sh.wn[wv] = c;
  __syncthreads();
  uint32_t s = 0;
#pragma unroll
  for (int u = 0; u < W; ++u) s += sh.wn[u];
  __syncthreads();
  return s;
}
// Min and max over the workgroup of per-lane values (NaN-free).
template <int W>
__device__ __forceinline__ void rows_block_minmax(float& mn, float& mx, RowSelLds<W>& sh, int wv,
                                                  int l) {
  mn = wave_ext_dpp<false>(mn);
  mx = wave_ext_dpp<true>(mx);
  if (l == 0) {
    sh.wmn[wv] = mn;
    sh.wmx[wv] = mx;
  }
  __syncthreads();
  mn = sh.wmn[0];
  mx = sh.wmx[0];
#pragma unroll
  for (int u = 1; u < W; ++u) {
    mn = fminf(mn, sh.wmn[u]);
    mx = fmaxf(mx, sh.wmx[u]);
  }
  __syncthreads();
}

// K-th largest of the candidates v (NaN: not a candidate), given their min
// lo and max hi and 1 <= K < their count. The histogram bins are cleared on
// entry.
template <int RW, int W>
__device__ RowThreshold rows_threshold(const float (&v)[RW], float lo, float hi, int krem,
                                       RowSelLds<W>& sh, int wv, int l) {
  constexpr int NT = 64 * W, NB = kRowBins;
  constexpr int BPT = NB / NT;  // bins per thread in the search for beta
  static_assert(NB % NT == 0, "bins per thread");
  for (int level = 0; level < kRowLevels; ++level) {
    if (lo == hi) return RowThreshold{lo, krem, false};
    const float half_w = hi * 0.5f - lo * 0.5f;
    if (!(half_w > 0.0f)) break;
    // bin of x in [lo, hi]: monotone in x, and (x/2 - lo/2) <= half_w keeps
    // the product at most NB (1 + 2^-23) without overflow
    const float scale = static_cast<float>(NB) / half_w;
    const float lo_h = lo * 0.5f;
    auto binof_at = [](float x, float lo_h, float scale) {
      const int b = cvt_i32_nan0(__builtin_fmaf(x, 0.5f, -lo_h) * scale);
      return b < NB - 1 ? b : NB - 1;
    };
    auto binof = [&](float x) { return binof_at(x, lo_h, scale); };
    if (level == 0) {
      // every candidate is in [lo, hi]; a non-candidate (NaN) lands in bin 0,
      // which is only ever the bin of the K-th largest when all candidates
      // above it number fewer than K: then the exact passes below, which
      // skip NaN, take over (see the count check)
#pragma unroll
      for (int i = 0; i < RW; ++i) atomicAdd(&sh.hist[binof(v[i])], 1u);
    } else {
#pragma unroll
      for (int i = 0; i < RW; ++i) {
        const float x = v[i];
        if (x >= lo && x <= hi) atomicAdd(&sh.hist[binof(x)], 1u);
      }
    }
    __syncthreads();
    // Thread t owns bins NB - BPT(t+1) .. NB - BPT t - 1: thread 0 the top
    // ones. Candidates above a thread's bins: the counts of the threads
    // before it (one scan per wave, one exchange of the wave totals).
    const int b0 = NB - BPT * (static_cast<int>(threadIdx.x) + 1);
    uint32_t h[BPT];
    uint32_t local = 0;
#pragma unroll
    for (int b = 0; b < BPT; ++b) {
      h[b] = sh.hist[b0 + b];
      local += h[b];
    }
    const uint32_t inc = wave_scan_dpp(local);
    if (l == 63) sh.part[wv] = inc;
    __syncthreads();
    uint32_t acc = inc - local;
#pragma unroll
    for (int u = 0; u < W; ++u) acc += u < wv ? sh.part[u] : 0u;
    const uint32_t kr = static_cast<uint32_t>(krem);
#pragma unroll
    for (int b = BPT - 1; b >= 0; --b) {
      if (acc < kr && acc + h[b] >= kr) {
        sh.beta = b0 + b;
        sh.above = acc;
        sh.hbeta = h[b];
      }
      acc += h[b];
    }
    __syncthreads();
    const int beta = sh.beta;
    krem -= static_cast<int>(sh.above);
    const uint32_t hbeta = sh.hbeta;
    // candidates of bin beta: x in [lo, hi] with binof(x) == beta, each
    // pass with its own copies of the parameters
    auto in_beta_fn = [&]() {
      const float clo = fresh(lo), chi = fresh(hi), clh = fresh(lo_h), csc = fresh(scale);
      const int cb = fresh(beta);
      return [=](float x) { return x >= clo && x <= chi && binof_at(x, clh, csc) == cb; };
    };
    if (hbeta <= static_cast<uint32_t>(kRowList)) {
      // ---- the bin's candidates to LDS, this wave's at list[wv]. A value
      // window of the bin widened by two bins on each side (far more than
      // the rounding of its ends) selects the rows that need the exact test.
      const float wbin = 2.0f * half_w / static_cast<float>(NB);
      const float wa = lo + static_cast<float>(beta - 2) * wbin;
      const float wb = lo + static_cast<float>(beta + 3) * wbin;
      uint32_t nl = 0;
      const auto in_beta = in_beta_fn();
#pragma unroll
      for (int i = 0; i < RW; ++i) {
        const float x = v[i];
        if (__ballot(x >= wa && x <= wb) != 0ull) {
          const bool in = in_beta(x);
          const uint64_t bm = __ballot(in);
          const uint32_t at = nl + lanes_below(bm);
          if (in && at < static_cast<uint32_t>(kRowList)) sh.list[wv][at] = x;
          nl += static_cast<uint32_t>(__popcll(bm));
        }
      }
      if (l == 0) sh.nlist[wv] = nl;
      __syncthreads();
      int total = 0;
#pragma unroll
      for (int u = 0; u < W; ++u) total += static_cast<int>(sh.nlist[u]);
      // All of the bin's candidates were found (a NaN counted in bin 0, or
      // a window too narrow for the rounding of values far from zero, would
      // leave fewer; all waves see the same total): rank them.
      if (total == static_cast<int>(hbeta)) {
        // lane j takes candidate j of the bin and counts the candidates above
        // it and equal to it; the krem-th largest has gt < krem <= gt + eq
        float x = __uint_as_float(0x7fc00000u);
        int off = 0;
#pragma unroll
        for (int u = 0; u < W; ++u) {
          const int nu = static_cast<int>(sh.nlist[u]);
          if (l >= off && l < off + nu) x = sh.list[u][l - off];
          off += nu;
        }
        uint32_t gt = 0, eq = 0;
        for (int j = 0; j < total; ++j) {
          const float y = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), j));
          gt += y > x ? 1u : 0u;
          eq += y == x ? 1u : 0u;
        }
        const uint32_t kq = static_cast<uint32_t>(krem);
        const uint64_t hit = __ballot(l < total && gt < kq && gt + eq >= kq);
        const int ls = static_cast<int>(__builtin_ctzll(hit));
        const float T = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), ls));
        const int gts = __builtin_amdgcn_readlane(static_cast<int>(gt), ls);
        const int eqs = __builtin_amdgcn_readlane(static_cast<int>(eq), ls);
        // every candidate equal to T is in this bin: eqs of them in all
        return RowThreshold{T, krem - gts, krem - gts == eqs};
      }
    }
    // ---- the bin's own range
    float bmn = INFINITY, bmx = -INFINITY;
    const auto in_beta = in_beta_fn();
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      const float x = v[i];
      if (in_beta(x)) {
        bmn = fminf(bmn, x);
        bmx = fmaxf(bmx, x);
      }
    }
    rows_block_minmax<W>(bmn, bmx, sh, wv, l);
    lo = bmn;
    hi = bmx;
    // clear the bins for the next level (every read of them is behind the
    // barriers of the min/max exchange)
#pragma unroll
    for (int b = 0; b < BPT; ++b) sh.hist[threadIdx.x * BPT + b] = 0u;
    __syncthreads();
  }
  if (lo == hi) return RowThreshold{lo, krem, false};
  // Exact bisection on order keys within [lo, hi]: the largest key x with
  // count(values in [x, hi]) >= krem.
  uint32_t klo = order_key(lo), khi = order_key(hi);
  while (klo < khi) {
    const uint32_t mid = klo + ((khi - klo + 1u) >> 1);
    const float fm = key_value(mid);
    uint32_t c = 0;
    const float chi = fresh(hi);
#pragma unroll
    for (int i = 0; i < RW; ++i) c += row_count(v[i] >= fm && v[i] <= chi);
    const uint32_t tot = rows_block_sum<W>(c, sh, wv, l);
    if (tot >= static_cast<uint32_t>(krem)) klo = mid; else khi = mid - 1u;
  }
  const float T = key_value(klo);
  uint32_t c = 0;
  const float chi = fresh(hi);
#pragma unroll
  for (int i = 0; i < RW; ++i) c += row_count(v[i] > T && v[i] <= chi);
  const uint32_t tgt = rows_block_sum<W>(c, sh, wv, l);
  return RowThreshold{T, krem - static_cast<int>(tgt), false};
}

// The register budget allows 6 waves per SIMD (80 VGPRs; 78 used at RW =
// 32): the kernel waits on loads, barriers and LDS atomics, so more resident
// workgroups hide more of it (64K: 1.567 -> 1.499 ms for the token select
// at 5 -> 6; at 7 the 32-row form spills).
template <int RW, int W>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(6, 8))) void
token_topk_rows_kernel(const float* __restrict__ scores, const int32_t* __restrict__ block_idx,
                       const int32_t* __restrict__ q_pos, int m, int B, int k, int L,
                       int32_t* __restrict__ token_idx, float* __restrict__ token_scores) {
  constexpr int NT = 64 * W, NB = kRowBins;
  __shared__ RowSelLds<W> sh;
  extern __shared__ uint4 stage[];  // k ids, then k scores when asked for
  const int64_t qi = blockIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l = threadIdx.x & 63;
  const int t = min(max(q_pos[qi], 0), L - 1);
  const int nblk = (L + B - 1) / B;
  const int lrpb = __builtin_ctz(B >> 6);  // log2 of the rows per slot (B = 64, 128, 256)
  const int nrows = (m * B) >> 6;
  const float* row = scores + qi * static_cast<int64_t>(m) * B;
  const float qnan = __uint_as_float(0x7fc00000u);
#pragma unroll
  for (int b = 0; b < NB / NT; ++b) sh.hist[threadIdx.x * (NB / NT) + b] = 0u;
  // Row r0 + j of this wave, in lane j < RW: its first token rbase (-1 for a
  // row without candidates: past the last row, an empty slot, a block past
  // the end of the keys) and rlim, the last lane that is a candidate (token
  // rbase + lane <= t), -1 for none.
  const int r0 = RW * wv;
  int rbase = -1;
  {
    const int r = r0 + l;
    const int c = l < RW && r < nrows ? block_idx[qi * m + (r >> lrpb)] : -1;
    if (c >= 0 && c < nblk) rbase = c * B + (r & ((1 << lrpb) - 1)) * 64;
  }
  const int rlim = rbase >= 0 ? min(t - rbase, 63) : -1;
  // the rows, all loads issued before any is used, from one lane address
  // with immediate row offsets (rows past the query's last are read from the
  // buffer's slack or the next query and masked)
  static_assert(RW * W <= 256, "rows per query within the buffer's slack");
  float v[RW];
  {
    const float* lrow = row + static_cast<int64_t>(r0) * 64 + l;
#pragma unroll
    for (int i = 0; i < RW; ++i) v[i] = lrow[i * 64];
  }
  // rows that are not whole candidates (usually only the query's own block)
  if (__ballot(l < RW && rlim < 63) != 0ull) {
#pragma unroll
    for (int i = 0; i < RW; ++i) v[i] = l <= __builtin_amdgcn_readlane(rlim, i) ? v[i] : qnan;
  }
  // ---- count, min and max of the candidates
  const uint32_t nw = wave_sum_dpp(static_cast<uint32_t>(max(rlim + 1, 0)));
  float mn = INFINITY, mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < RW; ++i) {
    mn = min_skip_nan(mn, v[i]);
    mx = max_skip_nan(mx, v[i]);
  }
  mn = wave_ext_dpp<false>(mn);
  mx = wave_ext_dpp<true>(mx);
  if (l == 0) {
    sh.wmn[wv] = mn;
    sh.wmx[wv] = mx;
    sh.wn[wv] = nw;
  }
  __syncthreads();
  uint32_t n = 0;
  float lo = sh.wmn[0], hi = sh.wmx[0];
#pragma unroll
  for (int u = 0; u < W; ++u) {
    n += sh.wn[u];
    lo = fminf(lo, sh.wmn[u]);
    hi = fmaxf(hi, sh.wmx[u]);
  }
  __syncthreads();
  const RowThreshold th = n <= static_cast<uint32_t>(k)
                              ? RowThreshold{-INFINITY, 0x7fffffff, true}
                              : rows_threshold<RW, W>(v, lo, hi, k, sh, wv, l);
  // ---- compaction: this wave's counts, then the waves before it; the kept
  // ids (and scores) are ranked into LDS and written out with 16-byte stores
  int32_t* sid = reinterpret_cast<int32_t*>(stage);
  float* ssc = token_scores ? reinterpret_cast<float*>(stage) + k : nullptr;
  uint32_t kept_all, kept;
  if (th.all) {
    // every candidate >= T is kept
    uint32_t gew = 0;
#pragma unroll
    for (int i = 0; i < RW; ++i) gew += row_count(v[i] >= th.T);
    if (l == 0) sh.wcnt[0][wv] = gew;
    __syncthreads();
    uint32_t before = 0, all = 0;
#pragma unroll
    for (int u = 0; u < W; ++u) {
      before += u < wv ? sh.wcnt[0][u] : 0u;
      all += sh.wcnt[0][u];
    }
    kept_all = all;
    kept = before;
    const float T = fresh(th.T);
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      const float x = v[i];
      const bool keep = x >= T;
      const uint64_t km = __ballot(keep);
      if (km != 0ull) {
        const uint32_t pos = kept + lanes_below(km);
        if (keep && pos < static_cast<uint32_t>(k)) {
          sid[pos] = __builtin_amdgcn_readlane(rbase, i) + l;
          if (ssc) ssc[pos] = x;
        }
        kept += static_cast<uint32_t>(__popcll(km));
      }
    }
  } else {
    // only the first `need` candidates equal to T (in position order)
    const uint32_t need = static_cast<uint32_t>(th.need);
    uint32_t gtw = 0, eqw = 0;
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      gtw += row_count(v[i] > th.T);
      eqw += row_count(v[i] == th.T);
    }
    if (l == 0) {
      sh.wcnt[0][wv] = gtw;
      sh.wcnt[1][wv] = eqw;
    }
    __syncthreads();
    uint32_t gtb = 0, ties = 0, gta = 0, tia = 0;
#pragma unroll
    for (int u = 0; u < W; ++u) {
      gtb += u < wv ? sh.wcnt[0][u] : 0u;
      ties += u < wv ? sh.wcnt[1][u] : 0u;
      gta += sh.wcnt[0][u];
      tia += sh.wcnt[1][u];
    }
    kept_all = gta + min(tia, need);
    kept = gtb + min(ties, need);
    const float T = fresh(th.T);
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      const float x = v[i];
      const uint64_t em = __ballot(x == T);
      bool keep;
      if (em == 0ull) {
        keep = x > T;
      } else {
        keep = x > T || (x == T && ties + lanes_below(em) < need);
        ties += static_cast<uint32_t>(__popcll(em));
      }
      const uint64_t km = __ballot(keep);
      if (km != 0ull) {
        const uint32_t pos = kept + lanes_below(km);
        if (keep && pos < static_cast<uint32_t>(k)) {
          sid[pos] = __builtin_amdgcn_readlane(rbase, i) + l;
          if (ssc) ssc[pos] = x;
        }
        kept += static_cast<uint32_t>(__popcll(km));
      }
    }
  }
  __syncthreads();
  int32_t* oi = token_idx + qi * k;
  float* os = token_scores ? token_scores + qi * k : nullptr;
  if ((k & 3) == 0) {
    for (int i = 4 * static_cast<int>(threadIdx.x); i < k; i += 4 * NT) {
      int4 o;
      o.x = i + 0 < static_cast<int>(kept_all) ? sid[i + 0] : -1;
      o.y = i + 1 < static_cast<int>(kept_all) ? sid[i + 1] : -1;
      o.z = i + 2 < static_cast<int>(kept_all) ? sid[i + 2] : -1;
      o.w = i + 3 < static_cast<int>(kept_all) ? sid[i + 3] : -1;
      *reinterpret_cast<int4*>(oi + i) = o;
      if (os) {
        float4 f;
        f.x = i + 0 < static_cast<int>(kept_all) ? ssc[i + 0] : qnan;
        f.y = i + 1 < static_cast<int>(kept_all) ? ssc[i + 1] : qnan;
        f.z = i + 2 < static_cast<int>(kept_all) ? ssc[i + 2] : qnan;
        f.w = i + 3 < static_cast<int>(kept_all) ? ssc[i + 3] : qnan;
        *reinterpret_cast<float4*>(os + i) = f;
      }
    }
  } else {
    for (int i = static_cast<int>(threadIdx.x); i < k; i += NT) {
      oi[i] = i < static_cast<int>(kept_all) ? sid[i] : -1;
      if (os) os[i] = i < static_cast<int>(kept_all) ? ssc[i] : qnan;
    }
  }
}

// below this many queries the row top-k uses kWideW waves per query
constexpr int64_t kFewQueries = 1024;
constexpr int kWideW = 16;

hipError_t launch_token_select(const uint16_t* qidx, Str3 qs, const uint16_t* kidx, Str3 ks,
                              const int32_t* q_pos, const int32_t* block_idx, int batch, int nq,
                              int L, int d, int B, int m, int k, int32_t* token_idx,
                              float* token_scores, void* ws, hipStream_t s) {
  const int nblk = (L + B - 1) / B;
  const int nkeys = batch * nblk;
  const size_t npairs = static_cast<size_t>(batch) * nq * m;
  const size_t max_tiles = (npairs + kTQ - 1) / kTQ + nkeys;
  TokWs w = carve(ws, batch, nq, L, B, m, nullptr);
  // Pairs are scored in place, without bucketing them by key block, when
  // there is one query per sequence (no key block has two pairs) or when
  // reading every pair's block directly gathers little (<= 256 MB, served
  // from L2 and the Infinity Cache): the bucketing's launches then cost more
  // than the reads they save.
  const bool direct =
      nq == 1 || npairs * static_cast<size_t>(B) * d * 2 <= (static_cast<size_t>(256) << 20);
  if (!direct) {
    const hipError_t e = launch_pair_buckets(block_idx, batch, nq, m, nblk, w, s);
    if (e != hipSuccess) return e;
  }
  const uint32_t np32 = static_cast<uint32_t>(npairs);
#define HISA_TS(D_, B_)                                                                       \
  do {                                                                                        \
    if (direct)                                                                               \
      hipLaunchKernelGGL((token_score_direct_kernel<D_, B_>),                                 \
                         dim3(static_cast<unsigned>((npairs * (B_ / 32) + 3) / 4)), dim3(256), \
                         0, s, qidx, qs.b, qs.t, kidx, ks.b, ks.t, L, nq, m, nblk, block_idx,  \
                         w.scores, np32);                                                     \
    else                                                                                      \
      hipLaunchKernelGGL((token_score_kernel<D_, B_>), dim3(static_cast<unsigned>(max_tiles)),  \
                         dim3(256), 0, s, qidx, qs.b, qs.t, kidx, ks.b, ks.t, L, nq, m, nblk,  \
                         w.tiles, w.total, w.tile_off, w.offs, w.cnt, w.pairs, w.scores);      \
  } while (0)
  if (d == 64) {
    if (B == 64) HISA_TS(64, 64); else if (B == 128) HISA_TS(64, 128); else HISA_TS(64, 256);
  } else {
    if (B == 64) HISA_TS(128, 64); else if (B == 128) HISA_TS(128, 128); else HISA_TS(128, 256);
  }
#undef HISA_TS
  const int64_t nq_total = static_cast<int64_t>(batch) * nq;
  const size_t stage_bytes = static_cast<size_t>(k) * 4 * (token_scores ? 2 : 1);
  if (B % 64 == 0 && m * B <= 16384 && m <= 256 && stage_bytes <= 65536) {
    const int nrows = m * B / 64;
    const dim3 gr(static_cast<unsigned>(nq_total));
#define HISA_TR(R_, W_)                                                                        \
  do {                                                                                        \
    hipLaunchKernelGGL((token_topk_rows_kernel<R_, W_>), gr, dim3(64 * W_), stage_bytes, s,    \
                       w.scores, block_idx, q_pos, m, B, k, L, token_idx, token_scores);      \
  } while (0)
    if (nq_total < kFewQueries) {
      // few queries (decode): kWideW waves per query, so that the CUs that get
      // a workgroup hold enough waves to hide the latency of each step
      const int rw = (nrows + kWideW - 1) / kWideW;  // rows per wave
      if (rw <= 2) HISA_TR(2, kWideW);
      else if (rw <= 4) HISA_TR(4, kWideW);
      else if (rw <= 8) HISA_TR(8, kWideW);
      else HISA_TR(16, kWideW);
    } else if (nrows > 128) {
      // more than 8192 candidates: 8 waves of up to 32 rows
      HISA_TR(32, 8);
    } else {
      const int rw = (nrows + 3) / 4;
      if (rw <= 2) HISA_TR(2, 4);
      else if (rw <= 4) HISA_TR(4, 4);
      else if (rw <= 8) HISA_TR(8, 4);
      else if (rw <= 16) HISA_TR(16, 4);
      else HISA_TR(32, 4);
    }
#undef HISA_TR
    return hipGetLastError();
  }
  const int items = (m * B + 255) / 256;
  dim3 g(static_cast<unsigned>(static_cast<size_t>(batch) * nq));
#define HISA_TK(I_)                                                                          \
  hipLaunchKernelGGL((token_topk_kernel<I_>), g, dim3(256), 0, s, w.scores, block_idx, q_pos, m, \
                     B, k, L, token_idx, token_scores)
  if (items <= 2) HISA_TK(2);
  else if (items <= 4) HISA_TK(4);
  else if (items <= 8) HISA_TK(8);
  else if (items <= 16) HISA_TK(16);
  else if (items <= 32) HISA_TK(32);
  else HISA_TK(64);
#undef HISA_TK
  return hipGetLastError();
}

// ------------------------------------------------------------ flat path
// Dense causal scoring: workgroup tile = 128 keys x 64 queries, wave w owns
// 32 keys. Rows of the score buffer have stride ldw = round_up(L, 4); only
// keys j <= t are read back by the selection.
template <int D>
__global__ __launch_bounds__(256) void flat_score_kernel(
    const uint16_t* __restrict__ qidx, int64_t qsb, int64_t qst, const uint16_t* __restrict__ kidx,
    int64_t ksb, int64_t kst, const int32_t* __restrict__ q_pos, int L, int nq, int64_t ldw,
    float* __restrict__ scores) {
  constexpr int KS = D / 32;
  const int b = blockIdx.z;
  const int j0 = blockIdx.x * 128, q0 = blockIdx.y * 64;
  const int wave = threadIdx.x / kWave, lane = lane_id();
  const int g = lane / 16, r16 = lane % 16;
  // skip tiles entirely above every query of the tile
  int tmax = -1;
  for (int i = lane; i < 64; i += kWave) {
    const int qq = q0 + i;
    if (qq < nq) tmax = max(tmax, q_pos[static_cast<int64_t>(b) * nq + qq]);
  }
  tmax = static_cast<int>(wave_max(static_cast<float>(tmax)));
  if (j0 > tmax) return;
  bf16x8 a[2][KS];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int j = min(j0 + wave * 32 + mt * 16 + r16, L - 1);
    const uint16_t* kr = kidx + b * ksb + static_cast<int64_t>(j) * kst + 8 * g;
#pragma unroll
    for (int s = 0; s < KS; ++s) a[mt][s] = as_bf16x8(*reinterpret_cast<const uint4*>(kr + 32 * s));
  }
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int qq = q0 + nt * 16 + r16;
    const uint16_t* qr = qidx + b * qsb + static_cast<int64_t>(min(qq, nq - 1)) * qst + 8 * g;
    bf16x8 bq[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) bq[s] = as_bf16x8(*reinterpret_cast<const uint4*>(qr + 32 * s));
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < KS; ++s) acc = mfma16(a[mt][s], bq[s], acc);
      const int j = j0 + wave * 32 + mt * 16 + 4 * g;
      if (qq < nq && j < L) {
        float* dst = scores + (static_cast<int64_t>(b) * nq + qq) * ldw + j;
        *reinterpret_cast<f32x4*>(dst) = acc;  // ldw % 4 == 0, j % 4 == 0
      }
    }
  }
}

// One workgroup (1024 threads) per query streams its row in chunks of
// 16384 candidates (thread t owns 16 consecutive positions per chunk).
__global__ __launch_bounds__(1024) void flat_topk_kernel(const float* __restrict__ scores,
                                                         const int32_t* __restrict__ q_pos,
                                                         int64_t ldw, int L, int k,
                                                         int32_t* __restrict__ token_idx,
                                                         float* __restrict__ token_scores) {
  constexpr int NT = 1024, ITEMS = 16, NB = 2048, CH = NT * ITEMS;
  __shared__ SelectLds<NT, NB> sh;
  const int64_t qi = blockIdx.x;
  const int n = min(max(q_pos[qi], 0), L - 1) + 1;
  const float* row = scores + qi * ldw;
  const int nchunks = (n + CH - 1) / CH;
  auto get = [&](int c, int i, float& v) -> bool {
    const int p = c * CH + threadIdx.x * ITEMS + i;
    if (p >= n) return false;
    v = row[p];
    return true;
  };
  const Threshold th = select_threshold<NT, ITEMS, NB>(get, nchunks, k, sh);
  uint32_t kept = 0, ties = 0;
  int32_t* oi = token_idx + qi * k;
  float* os = token_scores ? token_scores + qi * k : nullptr;
  for (int c = 0; c < nchunks; ++c) {
    select_compact<NT, ITEMS, NB>(get, c, th, kept, ties, sh, [&](uint32_t pos, int i, float v) {
      oi[pos] = c * CH + threadIdx.x * ITEMS + i;
      if (os) os[pos] = v;
    });
  }
  for (int i = kept + threadIdx.x; i < k; i += NT) {
    oi[i] = -1;
    if (os) os[i] = __uint_as_float(0x7fc00000u);
  }
}

size_t flat_workspace(int batch, int nq, int L, int /*k*/) {
  const size_t ldw = (static_cast<size_t>(L) + 3) & ~static_cast<size_t>(3);
  return align256(static_cast<size_t>(batch) * nq * ldw * 4);
}

hipError_t launch_flat_topk(const uint16_t* qidx, Str3 qs, const uint16_t* kidx, Str3 ks,
                            const int32_t* q_pos, int batch, int nq, int L, int d, int k,
                            int32_t* token_idx, float* token_scores, void* ws, hipStream_t s) {
  const int64_t ldw = (static_cast<int64_t>(L) + 3) & ~static_cast<int64_t>(3);
  float* sc = static_cast<float*>(ws);
  dim3 grid((L + 127) / 128, (nq + 63) / 64, batch);
  if (d == 64)
    hipLaunchKernelGGL(flat_score_kernel<64>, grid, dim3(256), 0, s, qidx, qs.b, qs.t, kidx, ks.b,
                       ks.t, q_pos, L, nq, ldw, sc);
  else
    hipLaunchKernelGGL(flat_score_kernel<128>, grid, dim3(256), 0, s, qidx, qs.b, qs.t, kidx,
                       ks.b, ks.t, q_pos, L, nq, ldw, sc);
  hipLaunchKernelGGL(flat_topk_kernel, dim3(static_cast<unsigned>(static_cast<size_t>(batch) * nq)),
                     dim3(1024), 0, s, sc, q_pos, ldw, L, k, token_idx, token_scores);
  return hipGetLastError();
}

}  // namespace hisa
