// C ABI of libhisa: argument validation, status codes, thread-local error
// text and dispatch to the kernel launchers. Nothing is launched unless every
// check passes; a failed check leaves all outputs untouched.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/hisa.h"
#include "internal.h"

namespace {

thread_local std::string g_err;

hisa_status_t fail(hisa_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

hisa_status_t ok() {
  g_err.clear();
  return HISA_OK;
}

hisa_status_t hip_status(hipError_t e, const char* where) {
  if (e != hipSuccess) return fail(HISA_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
  return ok();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
hisa::Str3 s3(hisa_strides_t s) { return hisa::Str3{s.batch, s.token, s.head}; }
bool strides8(hisa_strides_t s) { return s.batch % 8 == 0 && s.token % 8 == 0 && s.head % 8 == 0; }
bool nonneg(hisa_strides_t s) { return s.batch >= 0 && s.token >= 0 && s.head >= 0; }

#define CHECK(cond, st, ...)                    \
  do {                                          \
    if (!(cond)) return fail(st, __VA_ARGS__);  \
  } while (0)

hisa_status_t check_block(int B) {
  CHECK(B == 64 || B == 128 || B == 256, HISA_ERR_UNSUPPORTED,
        "block size B=%d unsupported (64, 128 or 256)", B);
  return HISA_OK;
}
hisa_status_t check_d(int d) {
  CHECK(d == 64 || d == 128, HISA_ERR_UNSUPPORTED, "indexer dim d=%d unsupported (64 or 128)", d);
  return HISA_OK;
}
hisa_status_t check_bf16(const void* p, hisa_strides_t s, const char* name) {
  CHECK(aligned16(p), HISA_ERR_SHAPE, "%s must be 16-byte aligned", name);
  CHECK(nonneg(s) && strides8(s), HISA_ERR_SHAPE,
        "%s strides must be non-negative multiples of 8 elements", name);
  return HISA_OK;
}

}  // namespace

extern "C" {

const char* hisa_last_error(void) { return g_err.c_str(); }

int hisa_abi_version(void) { return 3; }

hisa_status_t hisa_block_summary(const void* kidx, hisa_strides_t ks, int batch, int L, int d,
                                 int B, const void* proj, float* summary, void* split,
                                 hisa_stream_t stream) {
  CHECK(kidx != nullptr, HISA_ERR_NULL, "kidx is NULL");
  CHECK(summary != nullptr || split != nullptr, HISA_ERR_NULL, "summary and split both NULL");
  CHECK(batch >= 1 && L >= 1, HISA_ERR_SHAPE, "batch=%d L=%d must be >= 1", batch, L);
  hisa_status_t st;
  if ((st = check_d(d)) != HISA_OK) return st;
  if ((st = check_block(B)) != HISA_OK) return st;
  if ((st = check_bf16(kidx, ks, "kidx")) != HISA_OK) return st;
  CHECK(proj == nullptr || aligned16(proj), HISA_ERR_SHAPE, "proj must be 16-byte aligned");
  CHECK(summary == nullptr || aligned16(summary), HISA_ERR_SHAPE, "summary must be 16-byte aligned");
  CHECK(split == nullptr || aligned16(split), HISA_ERR_SHAPE, "split must be 16-byte aligned");
  CHECK((L + B - 1) / B <= 2147483647 / batch, HISA_ERR_SHAPE, "too many blocks");
  return hip_status(hisa::launch_block_summary(static_cast<const uint16_t*>(kidx), s3(ks), batch,
                                               L, d, B, static_cast<const uint16_t*>(proj),
                                               summary, static_cast<uint16_t*>(split),
                                               (L + B - 1) / B, 0,
                                               static_cast<hipStream_t>(stream)),
                    "hisa_block_summary");
}

hisa_status_t hisa_block_summary_update(const void* kidx, hisa_strides_t ks, int batch, int L,
                                        int d, int B, const void* proj, float* summary,
                                        void* split, int n_rows_cap, int first_row,
                                        hisa_stream_t stream) {
  CHECK(kidx != nullptr, HISA_ERR_NULL, "kidx is NULL");
  CHECK(summary != nullptr || split != nullptr, HISA_ERR_NULL, "summary and split both NULL");
  CHECK(batch >= 1 && L >= 1, HISA_ERR_SHAPE, "batch=%d L=%d must be >= 1", batch, L);
  hisa_status_t st;
  if ((st = check_d(d)) != HISA_OK) return st;
  if ((st = check_block(B)) != HISA_OK) return st;
  if ((st = check_bf16(kidx, ks, "kidx")) != HISA_OK) return st;
  CHECK(proj == nullptr || aligned16(proj), HISA_ERR_SHAPE, "proj must be 16-byte aligned");
  CHECK(summary == nullptr || aligned16(summary), HISA_ERR_SHAPE, "summary must be 16-byte aligned");
  CHECK(split == nullptr || aligned16(split), HISA_ERR_SHAPE, "split must be 16-byte aligned");
  const int n_rows = (L + B - 1) / B;
  CHECK(n_rows_cap >= n_rows, HISA_ERR_SHAPE, "n_rows_cap=%d below ceil(L/B)=%d", n_rows_cap,
        n_rows);
  CHECK(first_row >= 0 && first_row < n_rows, HISA_ERR_SHAPE,
        "first_row=%d must be in [0, ceil(L/B)=%d)", first_row, n_rows);
  CHECK(n_rows_cap <= 2147483647 / batch, HISA_ERR_SHAPE, "too many blocks");
  return hip_status(hisa::launch_block_summary(static_cast<const uint16_t*>(kidx), s3(ks), batch,
                                               L, d, B, static_cast<const uint16_t*>(proj),
                                               summary, static_cast<uint16_t*>(split),
                                               n_rows_cap, first_row,
                                               static_cast<hipStream_t>(stream)),
                    "hisa_block_summary_update");
}

hisa_status_t hisa_block_score(const void* qidx, hisa_strides_t qs, const int32_t* q_pos,
                               int batch, int nq, const void* split, int n_rows, int d, int B,
                               float* block_scores, hisa_stream_t stream) {
  CHECK(qidx && q_pos && split && block_scores, HISA_ERR_NULL,
        "qidx, q_pos, split and block_scores are required");
  CHECK(batch >= 1 && nq >= 1 && n_rows >= 1, HISA_ERR_SHAPE,
        "batch=%d nq=%d n_rows=%d must be >= 1", batch, nq, n_rows);
  CHECK(n_rows <= 65535 * 64 && batch <= 65535, HISA_ERR_UNSUPPORTED, "grid too large");
  hisa_status_t st;
  if ((st = check_d(d)) != HISA_OK) return st;
  if ((st = check_block(B)) != HISA_OK) return st;
  if ((st = check_bf16(qidx, qs, "qidx")) != HISA_OK) return st;
  CHECK(aligned16(split), HISA_ERR_SHAPE, "split must be 16-byte aligned");
  return hip_status(hisa::launch_block_score(static_cast<const uint16_t*>(qidx), s3(qs), q_pos,
                                             batch, nq, static_cast<const uint16_t*>(split),
                                             n_rows, d, B, block_scores,
                                             static_cast<hipStream_t>(stream)),
                    "hisa_block_score");
}

hisa_status_t hisa_select_blocks(const float* block_scores, const int32_t* q_pos, int batch,
                                 int nq, int n_rows, int B, int m, int32_t* block_idx,
                                 hisa_stream_t stream) {
  CHECK(block_scores && q_pos && block_idx, HISA_ERR_NULL,
        "block_scores, q_pos and block_idx are required");
  CHECK(batch >= 1 && nq >= 1 && n_rows >= 1, HISA_ERR_SHAPE,
        "batch=%d nq=%d n_rows=%d must be >= 1", batch, nq, n_rows);
  CHECK(batch <= 65535, HISA_ERR_UNSUPPORTED, "batch too large");
  CHECK(m >= 2, HISA_ERR_UNSUPPORTED, "m=%d must be >= 2 (first and local block)", m);
  hisa_status_t st;
  if ((st = check_block(B)) != HISA_OK) return st;
  return hip_status(hisa::launch_select_blocks(block_scores, q_pos, batch, nq, n_rows, B, m,
                                               block_idx, static_cast<hipStream_t>(stream)),
                    "hisa_select_blocks");
}

size_t hisa_route_blocks_workspace_bytes(int batch, int nq, int n_rows, int m) {
  if (batch < 1 || nq < 1 || n_rows < 1 || m < 2) return 0;
  return hisa::route_split_workspace(batch, nq, n_rows, m);
}

hisa_status_t hisa_route_blocks(const void* qidx, hisa_strides_t qs, const int32_t* q_pos,
                                int batch, int nq, const void* split, int n_rows, int d, int B,
                                int m, int32_t* block_idx, void* workspace, size_t workspace_bytes,
                                hisa_stream_t stream) {
  CHECK(qidx && q_pos && split && block_idx, HISA_ERR_NULL,
        "qidx, q_pos, split and block_idx are required");
  CHECK(batch >= 1 && nq >= 1 && n_rows >= 1, HISA_ERR_SHAPE,
        "batch=%d nq=%d n_rows=%d must be >= 1", batch, nq, n_rows);
  CHECK(n_rows <= hisa::kRouteMaxRows ||
            (m <= hisa::kRouteStreamMaxM && n_rows <= hisa::kRouteStreamMaxRows),
        HISA_ERR_UNSUPPORTED,
        "n_rows=%d with m=%d: on chip up to %d rows, streamed up to m=%d and %d rows; use "
        "hisa_block_score and hisa_select_blocks",
        n_rows, m, hisa::kRouteMaxRows, hisa::kRouteStreamMaxM, hisa::kRouteStreamMaxRows);
  CHECK(static_cast<long long>(batch) * ((nq + 15) / 16) <= 0x7fffffffLL, HISA_ERR_UNSUPPORTED,
        "grid too large");
  CHECK(m >= 2, HISA_ERR_UNSUPPORTED, "m=%d must be >= 2 (first and local block)", m);
  hisa_status_t st;
  if ((st = check_d(d)) != HISA_OK) return st;
  if ((st = check_block(B)) != HISA_OK) return st;
  if ((st = check_bf16(qidx, qs, "qidx")) != HISA_OK) return st;
  CHECK(aligned16(split), HISA_ERR_SHAPE, "split must be 16-byte aligned");
  const size_t need = hisa::route_split_workspace(batch, nq, n_rows, m);
  if (workspace != nullptr && need > 0) {
    CHECK((reinterpret_cast<uintptr_t>(workspace) & 255u) == 0, HISA_ERR_WORKSPACE,
          "workspace must be 256-byte aligned");
    CHECK(workspace_bytes >= need, HISA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu",
          workspace_bytes, need);
  }
  return hip_status(hisa::launch_route_blocks(static_cast<const uint16_t*>(qidx), s3(qs), q_pos,
                                              batch, nq, static_cast<const uint16_t*>(split),
                                              n_rows, d, B, m, block_idx,
                                              need > 0 ? workspace : nullptr,
                                              static_cast<hipStream_t>(stream)),
                    "hisa_route_blocks");
}

size_t hisa_token_select_workspace_bytes(int batch, int nq, int L, int B, int m, int k) {
  if (batch < 1 || nq < 1 || L < 1 || B < 1 || m < 1) return 0;
  return hisa::token_select_workspace(batch, nq, L, B, m, k);
}

hisa_status_t hisa_token_select(const void* qidx, hisa_strides_t qs, const void* kidx,
                                hisa_strides_t ks, const int32_t* q_pos, const int32_t* block_idx,
                                int batch, int nq, int L, int d, int B, int m, int k,
                                int32_t* token_idx, float* token_scores, void* workspace,
                                size_t workspace_bytes, hisa_stream_t stream) {
  CHECK(qidx && kidx && q_pos && block_idx && token_idx, HISA_ERR_NULL,
        "qidx, kidx, q_pos, block_idx and token_idx are required");
  CHECK(batch >= 1 && nq >= 1 && L >= 1, HISA_ERR_SHAPE, "batch=%d nq=%d L=%d must be >= 1",
        batch, nq, L);
  hisa_status_t st;
  if ((st = check_d(d)) != HISA_OK) return st;
  if ((st = check_block(B)) != HISA_OK) return st;
  CHECK(m >= 2 && static_cast<long>(m) * B <= 16384, HISA_ERR_UNSUPPORTED,
        "m=%d must be >= 2 with m*B <= 16384", m);
  CHECK(k >= 1 && k <= 16384, HISA_ERR_UNSUPPORTED, "k=%d must be in [1, 16384]", k);
  CHECK(static_cast<long long>(batch) * nq * m < 2147483647LL, HISA_ERR_UNSUPPORTED,
        "batch*nq*m too large");
  if ((st = check_bf16(qidx, qs, "qidx")) != HISA_OK) return st;
  if ((st = check_bf16(kidx, ks, "kidx")) != HISA_OK) return st;
  CHECK(workspace != nullptr, HISA_ERR_WORKSPACE, "workspace is NULL");
  CHECK((reinterpret_cast<uintptr_t>(workspace) & 255u) == 0, HISA_ERR_WORKSPACE,
        "workspace must be 256-byte aligned");
  const size_t need = hisa::token_select_workspace(batch, nq, L, B, m, k);
  CHECK(workspace_bytes >= need, HISA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu",
        workspace_bytes, need);
  CHECK(aligned16(token_idx), HISA_ERR_SHAPE, "token_idx must be 16-byte aligned");
  return hip_status(hisa::launch_token_select(static_cast<const uint16_t*>(qidx), s3(qs),
                                              static_cast<const uint16_t*>(kidx), s3(ks), q_pos,
                                              block_idx, batch, nq, L, d, B, m, k, token_idx,
                                              token_scores, workspace,
                                              static_cast<hipStream_t>(stream)),
                    "hisa_token_select");
}

hisa_status_t hisa_token_select_noalloc(const void* qidx, hisa_strides_t qs, const void* kidx,
                                        hisa_strides_t ks, const int32_t* q_pos,
                                        const int32_t* block_idx, int batch, int nq, int L, int d,
                                        int B, int m, int k, int32_t* token_idx,
                                        float* token_scores, hisa_stream_t stream) {
  static_assert(hisa::kNoallocScratchBytes == HISA_NOALLOC_SCRATCH_BYTES, "header limit");
  CHECK(qidx && kidx && q_pos && block_idx && token_idx, HISA_ERR_NULL,
        "qidx, kidx, q_pos, block_idx and token_idx are required");
  CHECK(batch >= 1 && nq >= 1 && L >= 1, HISA_ERR_SHAPE, "batch=%d nq=%d L=%d must be >= 1",
        batch, nq, L);
  hisa_status_t st;
  if ((st = check_d(d)) != HISA_OK) return st;
  if ((st = check_block(B)) != HISA_OK) return st;
  CHECK(m >= 2 && static_cast<long>(m) * B <= 16384, HISA_ERR_UNSUPPORTED,
        "m=%d must be >= 2 with m*B <= 16384", m);
  CHECK(k >= 1 && k <= 16384, HISA_ERR_UNSUPPORTED, "k=%d must be in [1, 16384]", k);
  CHECK(static_cast<long long>(batch) * nq * m < 2147483647LL, HISA_ERR_UNSUPPORTED,
        "batch*nq*m too large");
  if ((st = check_bf16(qidx, qs, "qidx")) != HISA_OK) return st;
  if ((st = check_bf16(kidx, ks, "kidx")) != HISA_OK) return st;
  CHECK(aligned16(token_idx), HISA_ERR_SHAPE, "token_idx must be 16-byte aligned");
  const size_t need = hisa::token_select_workspace(batch, nq, L, B, m, k);
  CHECK(need <= hisa::kNoallocScratchBytes, HISA_ERR_UNSUPPORTED,
        "this shape needs %zu bytes of scratch, above the fixed %zu of "
        "hisa_token_select_noalloc (use hisa_token_select with a workspace)",
        need, hisa::kNoallocScratchBytes);
  void* ws = nullptr;
  hisa_status_t hs = hip_status(hisa::noalloc_scratch(&ws), "hisa_token_select_noalloc scratch");
  if (hs != HISA_OK) return hs;
  return hip_status(hisa::launch_token_select(static_cast<const uint16_t*>(qidx), s3(qs),
                                              static_cast<const uint16_t*>(kidx), s3(ks), q_pos,
                                              block_idx, batch, nq, L, d, B, m, k, token_idx,
                                              token_scores, ws, static_cast<hipStream_t>(stream)),
                    "hisa_token_select_noalloc");
}

hisa_status_t hisa_auto_plan(int L, int B, int* hierarchical, int* m) {
  CHECK(hierarchical && m, HISA_ERR_NULL, "hierarchical and m are required");
  CHECK(L >= 1, HISA_ERR_SHAPE, "L=%d must be >= 1", L);
  hisa_status_t st;
  if ((st = check_block(B)) != HISA_OK) return st;
  *hierarchical = L >= 8192 ? 1 : 0;
  *m = std::min(std::max(64, L / 2000), 16384 / B);
  return HISA_OK;
}

size_t flat_indexer_topk_workspace_bytes(int batch, int nq, int L, int k) {
  if (batch < 1 || nq < 1 || L < 1) return 0;
  return hisa::flat_workspace(batch, nq, L, k);
}

hisa_status_t flat_indexer_topk(const void* qidx, hisa_strides_t qs, const void* kidx,
                                hisa_strides_t ks, const int32_t* q_pos, int batch, int nq, int L,
                                int d, int k, int32_t* token_idx, float* token_scores,
                                void* workspace, size_t workspace_bytes, hisa_stream_t stream) {
  CHECK(qidx && kidx && q_pos && token_idx, HISA_ERR_NULL,
        "qidx, kidx, q_pos and token_idx are required");
  CHECK(batch >= 1 && nq >= 1 && L >= 1, HISA_ERR_SHAPE, "batch=%d nq=%d L=%d must be >= 1",
        batch, nq, L);
  CHECK(batch <= 65535 && nq <= 65535 * 64, HISA_ERR_UNSUPPORTED, "grid too large");
  hisa_status_t st;
  if ((st = check_d(d)) != HISA_OK) return st;
  CHECK(k >= 1 && k <= 16384, HISA_ERR_UNSUPPORTED, "k=%d must be in [1, 16384]", k);
  if ((st = check_bf16(qidx, qs, "qidx")) != HISA_OK) return st;
  if ((st = check_bf16(kidx, ks, "kidx")) != HISA_OK) return st;
  CHECK(workspace != nullptr, HISA_ERR_WORKSPACE, "workspace is NULL");
  CHECK((reinterpret_cast<uintptr_t>(workspace) & 255u) == 0, HISA_ERR_WORKSPACE,
        "workspace must be 256-byte aligned");
  const size_t need = hisa::flat_workspace(batch, nq, L, k);
  CHECK(workspace_bytes >= need, HISA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu",
        workspace_bytes, need);
  return hip_status(hisa::launch_flat_topk(static_cast<const uint16_t*>(qidx), s3(qs),
                                           static_cast<const uint16_t*>(kidx), s3(ks), q_pos,
                                           batch, nq, L, d, k, token_idx, token_scores, workspace,
                                           static_cast<hipStream_t>(stream)),
                    "flat_indexer_topk");
}

size_t sparse_attn_fwd_workspace_bytes(int batch, int nq, int Hq, int Hkv, int Dk, int Dv,
                                       int topk) {
  if (batch < 1 || nq < 1 || Hq < 1 || Hkv < 1 || topk < 1 || Hq % Hkv != 0) return 0;
  return hisa::sparse_attn_workspace(batch, nq, Hq, Hkv, Dk, Dv, topk);
}

hisa_status_t sparse_attn_fwd(const void* q, hisa_strides_t qs, const void* k, hisa_strides_t ks,
                              const void* v, hisa_strides_t vs, int batch, int nq, int L, int Hq,
                              int Hkv, int Dk, int Dv, const int32_t* token_idx, int topk,
                              float scale, void* out, hisa_strides_t os, float* lse,
                              void* workspace, size_t workspace_bytes, hisa_stream_t stream) {
  CHECK(q && k && v && token_idx && out, HISA_ERR_NULL, "q, k, v, token_idx and out are required");
  CHECK(batch >= 1 && nq >= 1 && L >= 1 && topk >= 1 && Hq >= 1 && Hkv >= 1, HISA_ERR_SHAPE,
        "sizes must be >= 1");
  CHECK(Hq % Hkv == 0, HISA_ERR_SHAPE, "Hq=%d must be a multiple of Hkv=%d", Hq, Hkv);
  CHECK(Hq / Hkv <= 64, HISA_ERR_UNSUPPORTED, "at most 64 query heads per kv head");
  CHECK((Dk == 64 && Dv == 64) || (Dk == 128 && Dv == 128) || (Dk == 576 && Dv == 512),
        HISA_ERR_UNSUPPORTED, "(Dk, Dv)=(%d, %d) unsupported", Dk, Dv);
  CHECK(batch <= 65535 && Hkv <= 65535, HISA_ERR_UNSUPPORTED, "grid too large");
  hisa_status_t st;
  if ((st = check_bf16(q, qs, "q")) != HISA_OK) return st;
  if ((st = check_bf16(k, ks, "k")) != HISA_OK) return st;
  if ((st = check_bf16(v, vs, "v")) != HISA_OK) return st;
  if ((st = check_bf16(out, os, "out")) != HISA_OK) return st;
  CHECK(scale > 0.0f, HISA_ERR_SHAPE, "scale must be positive");
  if (workspace != nullptr) {
    CHECK((reinterpret_cast<uintptr_t>(workspace) & 255u) == 0, HISA_ERR_WORKSPACE,
          "workspace must be 256-byte aligned");
    const size_t need = hisa::sparse_attn_workspace(batch, nq, Hq, Hkv, Dk, Dv, topk);
    CHECK(workspace_bytes >= need, HISA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu",
          workspace_bytes, need);
  }
  return hip_status(hisa::launch_sparse_attn(static_cast<const uint16_t*>(q), s3(qs),
                                             static_cast<const uint16_t*>(k), s3(ks),
                                             static_cast<const uint16_t*>(v), s3(vs), batch, nq,
                                             L, Hq, Hkv, Dk, Dv, token_idx, topk, scale,
                                             static_cast<uint16_t*>(out), s3(os), lse, workspace,
                                             static_cast<hipStream_t>(stream)),
                    "sparse_attn_fwd");
}

size_t hils_two_level_attn_fwd_workspace_bytes(int batch, int H, int D, int m) {
  if (batch < 1 || H < 1 || (D != 64 && D != 128) || m < 2 || m > 64) return 0;
  return hisa::hils_workspace(batch, H, D, m);
}

hisa_status_t hils_two_level_attn_fwd(const void* q, hisa_strides_t qs, const void* k,
                                      hisa_strides_t ks, const void* v, hisa_strides_t vs,
                                      const float* khat, const int32_t* chunk_idx, int batch,
                                      int L, int H, int D, int C, int n_rows, int m,
                                      float scale_chunk, float scale_token, void* out,
                                      hisa_strides_t os, void* workspace, size_t workspace_bytes,
                                      hisa_stream_t stream) {
  CHECK(q && k && v && khat && chunk_idx && out, HISA_ERR_NULL,
        "q, k, v, khat, chunk_idx and out are required");
  CHECK(batch >= 1 && L >= 1 && H >= 1, HISA_ERR_SHAPE, "sizes must be >= 1");
  CHECK(D == 64 || D == 128, HISA_ERR_UNSUPPORTED, "D=%d unsupported (64 or 128)", D);
  hisa_status_t st;
  if ((st = check_block(C)) != HISA_OK) return st;
  CHECK(m >= 2 && m <= 64, HISA_ERR_UNSUPPORTED, "m=%d must be in [2, 64]", m);
  CHECK(n_rows == (L + C - 1) / C, HISA_ERR_SHAPE, "n_rows=%d must be ceil(L/C)", n_rows);
  CHECK(static_cast<long long>(batch) * H <= 2147483647LL, HISA_ERR_UNSUPPORTED, "grid too large");
  if ((st = check_bf16(k, ks, "k")) != HISA_OK) return st;
  if ((st = check_bf16(v, vs, "v")) != HISA_OK) return st;
  CHECK(nonneg(qs) && nonneg(os), HISA_ERR_SHAPE, "q/out strides must be non-negative");
  if (workspace != nullptr) {
    CHECK((reinterpret_cast<uintptr_t>(workspace) & 255u) == 0, HISA_ERR_WORKSPACE,
          "workspace must be 256-byte aligned");
    const size_t need = hisa::hils_workspace(batch, H, D, m);
    CHECK(workspace_bytes >= need, HISA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu",
          workspace_bytes, need);
  }
  return hip_status(hisa::launch_hils(static_cast<const uint16_t*>(q), s3(qs),
                                      static_cast<const uint16_t*>(k), s3(ks),
                                      static_cast<const uint16_t*>(v), s3(vs), khat, chunk_idx,
                                      batch, L, H, D, C, n_rows, m, scale_chunk, scale_token,
                                      static_cast<uint16_t*>(out), s3(os), workspace,
                                      static_cast<hipStream_t>(stream)),
                    "hils_two_level_attn_fwd");
}

size_t hils_two_level_prefill_fwd_workspace_bytes(int batch, int nq, int L, int H, int D, int C,
                                                  int m) {
  if (batch < 1 || nq < 1 || L < 1 || H < 1 || (D != 64 && D != 128) || m < 2 || m > 64 ||
      (C != 64 && C != 128 && C != 256))
    return 0;
  return hisa::hils_prefill_workspace(batch, nq, L, H, D, C, m);
}

hisa_status_t hils_two_level_prefill_fwd(const void* q, hisa_strides_t qs, const void* k,
                                         hisa_strides_t ks, const void* v, hisa_strides_t vs,
                                         const float* khat, const int32_t* chunk_idx,
                                         const void* proj, const int32_t* q_pos, int batch,
                                         int nq, int L, int H, int D, int C, int n_rows, int m,
                                         float scale_chunk, float scale_token, void* out,
                                         hisa_strides_t os, void* workspace,
                                         size_t workspace_bytes, hisa_stream_t stream) {
  CHECK(q && k && v && khat && chunk_idx && q_pos && out, HISA_ERR_NULL,
        "q, k, v, khat, chunk_idx, q_pos and out are required");
  CHECK(batch >= 1 && nq >= 1 && L >= 1 && H >= 1, HISA_ERR_SHAPE, "sizes must be >= 1");
  CHECK(D == 64 || D == 128, HISA_ERR_UNSUPPORTED, "D=%d unsupported (64 or 128)", D);
  hisa_status_t st;
  if ((st = check_block(C)) != HISA_OK) return st;
  CHECK(m >= 2 && m <= 64, HISA_ERR_UNSUPPORTED, "m=%d must be in [2, 64]", m);
  CHECK(n_rows == (L + C - 1) / C, HISA_ERR_SHAPE, "n_rows=%d must be ceil(L/C)", n_rows);
  CHECK(static_cast<long long>(batch) * H <= 65535LL, HISA_ERR_UNSUPPORTED,
        "batch*H=%lld exceeds 65535", static_cast<long long>(batch) * H);
  CHECK(static_cast<long long>(batch) * H * nq * m < (1LL << 32), HISA_ERR_UNSUPPORTED,
        "batch*H*nq*m must be below 2^32");
  if ((st = check_bf16(q, qs, "q")) != HISA_OK) return st;
  if ((st = check_bf16(k, ks, "k")) != HISA_OK) return st;
  if ((st = check_bf16(v, vs, "v")) != HISA_OK) return st;
  CHECK(aligned16(khat), HISA_ERR_SHAPE, "khat must be 16-byte aligned");
  CHECK(proj == nullptr || aligned16(proj), HISA_ERR_SHAPE, "proj must be 16-byte aligned");
  if ((st = check_bf16(out, os, "out")) != HISA_OK) return st;
  if (workspace != nullptr) {
    CHECK((reinterpret_cast<uintptr_t>(workspace) & 255u) == 0, HISA_ERR_WORKSPACE,
          "workspace must be 256-byte aligned");
    const size_t need = hisa::hils_prefill_workspace(batch, nq, L, H, D, C, m);
    CHECK(workspace_bytes >= need, HISA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu",
          workspace_bytes, need);
  }
  return hip_status(
      hisa::launch_hils_prefill(static_cast<const uint16_t*>(q), s3(qs),
                                static_cast<const uint16_t*>(k), s3(ks),
                                static_cast<const uint16_t*>(v), s3(vs), khat, chunk_idx,
                                static_cast<const uint16_t*>(proj), q_pos, batch, nq, L, H, D, C,
                                n_rows, m, scale_chunk, scale_token, static_cast<uint16_t*>(out),
                                s3(os), workspace, static_cast<hipStream_t>(stream)),
      "hils_two_level_prefill_fwd");
}

hisa_status_t hisa_gather_probe(const void* table, int64_t row_stride_bytes, int row_bytes,
                                int n_rows, const int32_t* ids, int nq, int topk, int waves,
                                int depth, int rot_ticks, hisa_stream_t stream) {
  CHECK(table && ids, HISA_ERR_NULL, "table and ids are required");
  CHECK(row_bytes == 256 || row_bytes == 1152, HISA_ERR_UNSUPPORTED,
        "row_bytes=%d unsupported (256 or 1152)", row_bytes);
  CHECK(waves == 4 || waves == 8, HISA_ERR_UNSUPPORTED, "waves=%d unsupported (4 or 8)", waves);
  CHECK(depth >= 1 && depth <= 4, HISA_ERR_UNSUPPORTED, "depth=%d must be in [1, 4]", depth);
  CHECK(rot_ticks >= 0, HISA_ERR_SHAPE, "rot_ticks=%d must be >= 0", rot_ticks);
  CHECK(n_rows >= 1 && nq >= 1 && topk >= 1, HISA_ERR_SHAPE, "sizes must be >= 1");
  CHECK(topk <= 4096, HISA_ERR_UNSUPPORTED, "topk=%d above 4096", topk);
  CHECK(nq <= 2147483647 - 7, HISA_ERR_UNSUPPORTED, "grid too large");
  CHECK(aligned16(table), HISA_ERR_SHAPE, "table must be 16-byte aligned");
  CHECK(row_stride_bytes >= row_bytes && row_stride_bytes % 16 == 0, HISA_ERR_SHAPE,
        "row_stride_bytes=%lld must be a multiple of 16 and >= row_bytes",
        static_cast<long long>(row_stride_bytes));
  return hip_status(hisa::launch_gather_probe(table, row_stride_bytes, row_bytes, n_rows, ids, nq,
                                              topk, waves, depth, rot_ticks,
                                              static_cast<hipStream_t>(stream)),
                    "hisa_gather_probe");
}

}  // extern "C"
