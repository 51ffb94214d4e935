// Launchers shared between the C ABI layer and the kernel files. Every
// launcher assumes its arguments were validated by the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace hisa {

struct Str3 {
  int64_t b, t, h;
};

// indexer.hip
// rows first_row .. ceil(L/B)-1 of tables with n_rows_cap rows per sequence
hipError_t launch_block_summary(const uint16_t* kidx, Str3 ks, int batch, int L, int d, int B,
                                const uint16_t* proj, float* summary, uint16_t* split,
                                int n_rows_cap, int first_row, hipStream_t s);
hipError_t launch_block_score(const uint16_t* qidx, Str3 qs, const int32_t* q_pos, int batch,
                              int nq, const uint16_t* split, int n_rows, int d, int B,
                              float* scores, hipStream_t s);
hipError_t launch_select_blocks(const float* scores, const int32_t* q_pos, int batch, int nq,
                                int n_rows, int B, int m, int32_t* block_idx, hipStream_t s);

// tokens.hip
size_t token_select_workspace(int batch, int nq, int L, int B, int m, int k);
hipError_t launch_token_select(const uint16_t* qidx, Str3 qs, const uint16_t* kidx, Str3 ks,
                              const int32_t* q_pos, const int32_t* block_idx, int batch, int nq,
                              int L, int d, int B, int m, int k, int32_t* token_idx,
                              float* token_scores, void* ws, hipStream_t s);
// the allocation-free token selection: the device address of the fixed
// scratch array on the current device (looked up on the first call there)
constexpr size_t kNoallocScratchBytes = static_cast<size_t>(64) << 20;
hipError_t noalloc_scratch(void** ptr);
size_t flat_workspace(int batch, int nq, int L, int k);
hipError_t launch_flat_topk(const uint16_t* qidx, Str3 qs, const uint16_t* kidx, Str3 ks,
                            const int32_t* q_pos, int batch, int nq, int L, int d, int k,
                            int32_t* token_idx, float* token_scores, void* ws, hipStream_t s);

// attention.hip; ws (may be null) holds at least sparse_attn_workspace() bytes
size_t sparse_attn_workspace(int batch, int nq, int Hq, int Hkv, int Dk, int Dv, int topk);
hipError_t launch_sparse_attn(const uint16_t* q, Str3 qs, const uint16_t* k, Str3 ks,
                              const uint16_t* v, Str3 vs, int batch, int nq, int L, int Hq,
                              int Hkv, int Dk, int Dv, const int32_t* token_idx, int topk,
                              float scale, uint16_t* out, Str3 os, float* lse, void* ws,
                              hipStream_t s);

// attention_d128.hip: head width 128, at most 16 query heads per kv head;
// with ws (attn_d128_workspace() bytes, 0 when it does not split) the token
// lists of few items are split over several waves
size_t attn_d128_workspace(int batch, int nq, int Hkv, int G, int topk);
hipError_t launch_attn_d128(const uint16_t* q, Str3 qs, const uint16_t* k, Str3 ks,
                            const uint16_t* v, Str3 vs, int batch, int nq, int L, int Hkv, int G,
                            const int32_t* token_idx, int topk, float scale, uint16_t* out,
                            Str3 os, float* lse, void* ws, hipStream_t s);

// attention_mla.hip: 64 query heads over one 576-wide latent row (V = first 512 columns)
hipError_t launch_mla_attn(const uint16_t* q, Str3 qs, const uint16_t* kv, Str3 ks, int batch,
                           int nq, int L, int Hkv, const int32_t* token_idx, int topk, float scale,
                           uint16_t* out, Str3 os, float* lse, hipStream_t s);

// indexer.hip: steps 2 and 3 fused (scores on chip when n_rows <= kRouteMaxRows,
// else streamed through per-query candidate buffers, which needs m - 2 <= 128)
constexpr int kRouteMaxRows = 64 * 16 + 2;
constexpr int kRouteStreamMaxM = 130;
constexpr int kRouteStreamMaxRows = 65537;  // candidate positions fit 16 bits
// with ws (route_split_workspace() bytes, 0 when the shape does not split)
// and fewer than 1024 queries, each query's blocks are scored and selected in
// parts over several workgroups and merged
size_t route_split_workspace(int batch, int nq, int n_rows, int m);
hipError_t launch_route_blocks(const uint16_t* qidx, Str3 qs, const int32_t* q_pos, int batch,
                               int nq, const uint16_t* split, int n_rows, int d, int B, int m,
                               int32_t* block_idx, void* ws, hipStream_t s);

// tokens.hip: (query, slot) entries of a [batch][nq][m] block list bucketed by
// (sequence, block), in tiles of kPairTile entries
constexpr int kPairTile = 64;
struct PairBuckets {
  uint32_t* cnt;        // [nkeys] entries per bucket
  uint32_t* cursor;     // [nkeys] scatter cursors
  uint32_t* offs;       // [nkeys] first entry of each bucket in pairs
  uint32_t* tile_off;   // [nkeys] first tile of each bucket
  uint32_t* total;      // [4]: entries, tiles
  uint32_t* part;       // scan partials
  uint32_t* pairs;      // [npairs] entry indices (b*nq + q)*m + slot, grouped by bucket
  uint32_t* tiles;      // [max tiles] bucket of each tile
};
PairBuckets carve_pair_buckets(void* ws, int batch, int nq, int m, int nblk, size_t* bytes);
hipError_t launch_pair_buckets(const int32_t* block_idx, int batch, int nq, int m, int nblk,
                               const PairBuckets& w, hipStream_t s);

// hils.hip; ws (may be null) holds at least hils_workspace() bytes (0 when the
// shape never splits its chunks over workgroups)
size_t hils_workspace(int batch, int H, int D, int m);
hipError_t launch_hils(const uint16_t* q, Str3 qs, const uint16_t* k, Str3 ks, const uint16_t* v,
                       Str3 vs, const float* khat, const int32_t* chunk_idx, int batch, int L,
                       int H, int D, int C, int n_rows, int m, float scale_chunk,
                       float scale_token, uint16_t* out, Str3 os, void* ws, hipStream_t s);

hipError_t launch_hils_prefill(const uint16_t* q, Str3 qs, const uint16_t* k, Str3 ks,
                               const uint16_t* v, Str3 vs, const float* khat,
                               const int32_t* chunk_idx, const uint16_t* proj,
                               const int32_t* q_pos, int batch, int nq, int L, int H, int D,
                               int C, int n_rows, int m, float scale_chunk, float scale_token,
                               uint16_t* out, Str3 os, void* ws, hipStream_t s);
size_t hils_prefill_workspace(int batch, int nq, int L, int H, int D, int C, int m);

// probe.hip: row_bytes 256 or 1152, waves 4 or 8, depth 1..4, topk <= 4096
hipError_t launch_gather_probe(const void* table, int64_t row_stride, int row_bytes, int n_rows,
                               const int32_t* ids, int nq, int topk, int waves, int depth,
                               int rot_ticks, hipStream_t s);

inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

}  // namespace hisa
