// Gather-rate probe: the memory side of the sparse attention kernels alone.
//
// The attention over the selected tokens (HISA explainer 1.1; HISA news
// article: the downstream attention is unchanged) reads, per query, the rows
// its token list names from a resident K/V table, straight into LDS with
// 16-byte direct loads, 8 lanes per 128-byte line. This kernel issues exactly
// that stream for given id lists and does nothing with the data, so its rate
// is the ceiling the gathers alone allow on this chip for those lists (the
// token selection of the explainer's section 1.3 is memory-side work of the
// same kind). The launch mirrors the attention: one workgroup per query,
// queries dealt to the eight XCDs in contiguous ranges, a ring of 32-row
// tiles in LDS, DEPTH tiles of loads in flight per wave.
#include "common.hpp"
#include "internal.h"

namespace hisa {
namespace probe {

typedef __attribute__((address_space(3))) void* lds_ptr;
typedef __attribute__((address_space(1))) void* glb_ptr;

constexpr int NT = 32;         // rows per tile
// s_waitcnt immediate that waits until at most n vector loads are in flight
// (vmcnt bits 3:0 and 15:14; the other counters left at their maxima)
constexpr int vmcnt_only(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }
constexpr int kMaxIds = 4096;  // ids per query staged in LDS

// LPR: 128-byte lines per row; W: waves; DEPTH: tiles in flight per wave.
// The ring holds min(DEPTH + 1, NBUF) tiles; nothing reads it, so a tile may
// land on a slot whose previous loads are still in flight.
// rot_ticks > 0: each query starts its sweep at tile (clock / rot_ticks) mod
// ntiles and wraps around, the clock being the constant-rate real-time
// counter read once per workgroup; queries running at the same time then read
// the same region of their (ascending) lists together whatever their start.
template <int LPR, int W, int DEPTH, int NBUF>
__global__ __launch_bounds__(64 * W) void gather_probe_kernel(const uint8_t* __restrict__ table,
                                                              int64_t row_stride, int n_rows,
                                                              const int32_t* __restrict__ ids,
                                                              int nq, int topk, int rot_ticks) {
  constexpr int IPT = NT * LPR / 8;       // 1 KB load instructions per tile
  constexpr int PER = (IPT + W - 1) / W;  // per wave (the last wave may issue fewer)
  static_assert(DEPTH * PER <= 62, "load counter range");
  __shared__ uint4 ring[NBUF][IPT * 64];
  __shared__ int sid[kMaxIds];
  __shared__ int s_first;
  const int per = (nq + 7) / 8;
  const int qi = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (qi >= nq) return;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), l = threadIdx.x & 63;
  const int32_t* qids = ids + static_cast<int64_t>(qi) * topk;
  for (int i = threadIdx.x; i < topk; i += 64 * W) {
    const int id = qids[i];
    sid[i] = static_cast<unsigned>(id) < static_cast<unsigned>(n_rows) ? id : 0;
  }
  const int ntiles = (topk + NT - 1) / NT;
  if (threadIdx.x == 0)
    s_first = rot_ticks > 0
                  ? static_cast<int>((__builtin_amdgcn_s_memrealtime() / rot_ticks) % ntiles)
                  : 0;
  __syncthreads();
  const int first = s_first;
  for (int i = 0; i < ntiles; ++i) {
    const int t = first + i < ntiles ? first + i : first + i - ntiles;
    uint4* dst = ring[i % NBUF];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int j = w + W * k;  // instruction of the tile
      if (j < IPT) {
        const int line = 8 * j + (l >> 3);
        const int r = line / LPR, c = line - r * LPR;
        const int row = sid[min(t * NT + r, topk - 1)];
        const uint8_t* src = table + static_cast<int64_t>(row) * row_stride + 128 * c + 16 * (l & 7);
        __builtin_amdgcn_global_load_lds((glb_ptr)src, (lds_ptr)(dst + 64 * j), 16, 0, 0);
      }
    }
    // at most DEPTH tiles of this wave's loads stay in flight
    __builtin_amdgcn_s_waitcnt(vmcnt_only(DEPTH * PER));
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
}

template <int LPR, int W, int DEPTH>
hipError_t launch(const uint8_t* table, int64_t stride, int n_rows, const int32_t* ids, int nq,
                  int topk, int rot, hipStream_t s) {
  constexpr int NBUF = (LPR == 9) ? ((DEPTH + 1) < 3 ? (DEPTH + 1) : 3) : (DEPTH + 1);
  const int per = (nq + 7) / 8;
  hipLaunchKernelGGL((gather_probe_kernel<LPR, W, DEPTH, NBUF>), dim3(8 * per), dim3(64 * W), 0,
                     s, table, stride, n_rows, ids, nq, topk, rot);
  return hipGetLastError();
}

}  // namespace probe

// row_bytes 256 (two lines) or 1152 (nine lines); waves 4 or 8; depth 1..4
hipError_t launch_gather_probe(const void* table, int64_t row_stride, int row_bytes, int n_rows,
                               const int32_t* ids, int nq, int topk, int waves, int depth,
                               int rot_ticks, hipStream_t s) {
  const uint8_t* t = static_cast<const uint8_t*>(table);
  if (row_bytes == 1152) {
    if (waves == 4) {
      if (depth == 1) return probe::launch<9, 4, 1>(t, row_stride, n_rows, ids, nq, topk, rot_ticks, s);
      if (depth == 2) return probe::launch<9, 4, 2>(t, row_stride, n_rows, ids, nq, topk, rot_ticks, s);
      if (depth == 3) return probe::launch<9, 4, 3>(t, row_stride, n_rows, ids, nq, topk, rot_ticks, s);
      return probe::launch<9, 4, 4>(t, row_stride, n_rows, ids, nq, topk, rot_ticks, s);
    }
    if (depth == 1) return probe::launch<9, 8, 1>(t, row_stride, n_rows, ids, nq, topk, rot_ticks, s);
    if (depth == 2) return probe::launch<9, 8, 2>(t, row_stride, n_rows, ids, nq, topk, rot_ticks, s);
    if (depth == 3) return probe::launch<9, 8, 3>(t, row_stride, n_rows, ids, nq, topk, rot_ticks, s);
    return probe::launch<9, 8, 4>(t, row_stride, n_rows, ids, nq, topk, rot_ticks, s);
  }
  if (waves == 4) {
    if (depth == 1) return probe::launch<2, 4, 1>(t, row_stride, n_rows, ids, nq, topk, rot_ticks, s);
    if (depth == 2) return probe::launch<2, 4, 2>(t, row_stride, n_rows, ids, nq, topk, rot_ticks, s);
    if (depth == 3) return probe::launch<2, 4, 3>(t, row_stride, n_rows, ids, nq, topk, rot_ticks, s);
    return probe::launch<2, 4, 4>(t, row_stride, n_rows, ids, nq, topk, rot_ticks, s);
  }
  if (depth == 1) return probe::launch<2, 8, 1>(t, row_stride, n_rows, ids, nq, topk, rot_ticks, s);
  if (depth == 2) return probe::launch<2, 8, 2>(t, row_stride, n_rows, ids, nq, topk, rot_ticks, s);
  if (depth == 3) return probe::launch<2, 8, 3>(t, row_stride, n_rows, ids, nq, topk, rot_ticks, s);
  return probe::launch<2, 8, 4>(t, row_stride, n_rows, ids, nq, topk, rot_ticks, s);
}

}  // namespace hisa
