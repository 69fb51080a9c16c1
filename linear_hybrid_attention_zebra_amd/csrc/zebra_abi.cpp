// C ABI of libzebra: argument validation, then kernel dispatch. Every check
// runs before the first HIP call, so a rejected call enqueues nothing.
#include "../../include/zebra.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <utility>
#include <vector>

#include "common.h"

namespace {

constexpr int32_t kMaxTileTokens = 1024;
constexpr int32_t kMaxKeyTiles = 32768;

struct Range {
  uintptr_t lo, hi;  // [lo, hi) in bytes; empty when lo == hi
};

bool seq_shape_ok(const zebra_seq& s) {
  return s.n_tokens >= 0 && s.n_heads >= 0 && s.stride_token >= 0 && s.stride_head >= 0;
}

bool seq_empty(const zebra_seq& s) { return s.n_tokens == 0 || s.n_heads == 0; }

Range seq_range(const void* p, const zebra_seq& s, size_t elem) {
  if (seq_empty(s) || p == nullptr) return {0, 0};
  const uintptr_t base = (uintptr_t)p;
  const uint64_t last = (uint64_t)(s.n_heads - 1) * (uint64_t)s.stride_head +
                        (uint64_t)(s.n_tokens - 1) * (uint64_t)s.stride_token +
                        (uint64_t)s.head_dim;
  return {base, base + (uintptr_t)(last * elem)};
}

Range flat_range(const void* p, uint64_t count, size_t elem) {
  if (p == nullptr || count == 0) return {0, 0};
  return {(uintptr_t)p, (uintptr_t)p + (uintptr_t)(count * elem)};
}

bool overlaps(Range a, Range b) {
  if (a.lo == a.hi || b.lo == b.hi) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

// An output sequence must not write one element twice: the (stride, extent)
// pairs of its three dimensions, sorted by stride, must nest. Only dimensions
// of extent > 1 are listed, so a zero stride among them always repeats
// elements (it sorts first, where the nesting test alone would pass it).
bool seq_self_disjoint(const zebra_seq& s) {
  if (seq_empty(s)) return true;
  std::vector<std::pair<int64_t, int64_t>> dims = {{1, s.head_dim}};
  if (s.n_tokens > 1) dims.push_back({s.stride_token, s.n_tokens});
  if (s.n_heads > 1) dims.push_back({s.stride_head, s.n_heads});
  std::sort(dims.begin(), dims.end());
  int64_t extent = 0;
  for (auto& d : dims) {
    if (d.first == 0 || d.first < extent) return false;
    extent = d.first * d.second;
  }
  return true;
}

// bf16 or f32 sequence with 16-byte aligned rows
zebra_status check_seq(const void* p, const zebra_seq& s, bool is_output) {
  if (!seq_shape_ok(s)) return ZEBRA_ERR_INVALID_ARG;
  if (s.head_dim != zebra::kHeadDim) return ZEBRA_ERR_UNSUPPORTED;
  if (seq_empty(s)) return ZEBRA_OK;
  if (p == nullptr) return ZEBRA_ERR_INVALID_ARG;
  if (((uintptr_t)p % 16) != 0 || (s.stride_token % 8) != 0 || (s.stride_head % 8) != 0)
    return ZEBRA_ERR_UNSUPPORTED;
  if (is_output && !seq_self_disjoint(s)) return ZEBRA_ERR_INVALID_ARG;
  return ZEBRA_OK;
}

zebra_status hip_status(hipError_t e) { return e == hipSuccess ? ZEBRA_OK : ZEBRA_ERR_HIP; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

static_assert(zebra::kSparseNoLandmarks == ZEBRA_SPARSE_NO_LANDMARKS, "flag bits");
static_assert(zebra::kSparseLandmarkLogCount == ZEBRA_SPARSE_LANDMARK_LOG_COUNT, "flag bits");

extern "C" {

const char* zebra_status_string(zebra_status status) {
  switch (status) {
    case ZEBRA_OK:
      return "ZEBRA_OK";
    case ZEBRA_ERR_INVALID_ARG:
      return "ZEBRA_ERR_INVALID_ARG: bad pointer, size, stride, overlap or top_k";
    case ZEBRA_ERR_UNSUPPORTED:
      return "ZEBRA_ERR_UNSUPPORTED: head_dim, tile size, alignment or length not implemented";
    case ZEBRA_ERR_WORKSPACE:
      return "ZEBRA_ERR_WORKSPACE: workspace smaller than the size query returned";
    case ZEBRA_ERR_HIP:
      return "ZEBRA_ERR_HIP: the HIP runtime rejected a launch";
  }
  return "unknown zebra_status";
}

const char* zebra_version(void) { return "zebra 0.1.0 (gfx950, ABI 1)"; }

zebra_status zebra_pool_landmarks(const void* x, zebra_seq xs, int32_t tile, float* mean_out,
                                  void* stream) {
  zebra_status st = check_seq(x, xs, false);
  if (st != ZEBRA_OK) return st;
  if (tile < 1) return ZEBRA_ERR_INVALID_ARG;
  if (tile > kMaxTileTokens) return ZEBRA_ERR_UNSUPPORTED;
  if (seq_empty(xs)) return ZEBRA_OK;
  if (mean_out == nullptr || ((uintptr_t)mean_out % 16) != 0) return ZEBRA_ERR_INVALID_ARG;
  const int64_t t = ceil_div(xs.n_tokens, tile);
  const Range out = flat_range(mean_out, (uint64_t)xs.n_heads * t * zebra::kHeadDim, 4);
  if (overlaps(out, seq_range(x, xs, 2))) return ZEBRA_ERR_INVALID_ARG;
  return hip_status(zebra::launch_pool((const uint16_t*)x, xs.n_tokens, xs.n_heads,
                                       xs.stride_token, xs.stride_head, tile, mean_out,
                                       (hipStream_t)stream));
}

size_t zebra_select_tiles_workspace(int32_t n_heads, int32_t t_q, int32_t t_k) {
  if (n_heads <= 0 || t_q <= 0 || t_k <= 0) return 0;
  return (size_t)n_heads * (size_t)t_q * (size_t)zebra::score_row_stride(t_k) * sizeof(float);
}

zebra_status zebra_select_tiles(const float* qbar, const float* kbar, int32_t n_heads,
                                int32_t t_q, int32_t t_k, int32_t head_dim, int32_t top_k,
                                int32_t* sel_out, void* workspace, size_t workspace_bytes,
                                void* stream) {
  if (n_heads < 0 || t_q < 0 || t_k < 0) return ZEBRA_ERR_INVALID_ARG;
  if (head_dim != zebra::kHeadDim) return ZEBRA_ERR_UNSUPPORTED;
  if (t_k > kMaxKeyTiles) return ZEBRA_ERR_UNSUPPORTED;
  if (n_heads == 0 || t_q == 0) return ZEBRA_OK;
  if (t_k == 0 || top_k < 1 || top_k > t_k) return ZEBRA_ERR_INVALID_ARG;
  if (qbar == nullptr || kbar == nullptr || sel_out == nullptr) return ZEBRA_ERR_INVALID_ARG;
  const size_t need = zebra_select_tiles_workspace(n_heads, t_q, t_k);
  if (workspace == nullptr || workspace_bytes < need) return ZEBRA_ERR_WORKSPACE;
  if (((uintptr_t)workspace % 16) != 0 || ((uintptr_t)qbar % 16) != 0 ||
      ((uintptr_t)kbar % 16) != 0 || ((uintptr_t)sel_out % 4) != 0)
    return ZEBRA_ERR_INVALID_ARG;
  const Range sel = flat_range(sel_out, (uint64_t)n_heads * t_q * top_k, 4);
  const Range ws = flat_range(workspace, need, 1);
  const Range qr = flat_range(qbar, (uint64_t)n_heads * t_q * head_dim, 4);
  const Range kr = flat_range(kbar, (uint64_t)n_heads * t_k * head_dim, 4);
  if (overlaps(sel, qr) || overlaps(sel, kr) || overlaps(sel, ws) || overlaps(ws, qr) ||
      overlaps(ws, kr))
    return ZEBRA_ERR_INVALID_ARG;
  return hip_status(zebra::launch_select(qbar, kbar, n_heads, t_q, t_k, top_k, sel_out,
                                         (float*)workspace, (hipStream_t)stream));
}

size_t zebra_tile_sparse_attn_workspace(int64_t n_q, int64_t n_kv, int32_t n_heads,
                                        int32_t head_dim, int32_t q_tile, int32_t k_tile,
                                        int32_t top_k) {
  if (n_q <= 0 || n_kv <= 0 || n_heads <= 0 || head_dim != zebra::kHeadDim) return 0;
  if (k_tile != 32 && k_tile != 64) return 0;
  if (q_tile != 32 && q_tile != 64 && q_tile != 128) return 0;
  if (top_k < 1) return 0;
  return zebra::sparse_workspace_bytes(n_q, n_kv, n_heads, q_tile, k_tile, top_k);
}

zebra_status zebra_tile_sparse_attn(const void* q, zebra_seq qs, const void* k, const void* v,
                                    zebra_seq kvs, const float* kbar, const float* vbar,
                                    const int32_t* sel, int32_t q_tile, int32_t k_tile,
                                    int32_t top_k, float scale, void* o, zebra_seq os,
                                    zebra_dtype o_dtype, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  return zebra_tile_sparse_attn_ex(q, qs, k, v, kvs, kbar, vbar, sel, q_tile, k_tile, top_k,
                                   scale, o, os, o_dtype, 0u, workspace, workspace_bytes, stream);
}

// zebra_tile_sparse_attn_ex and zebra_tile_sparse_attn_lse: lse_out (float32 [H][Nq]) or NULL
static zebra_status sparse_fwd(const void* q, zebra_seq qs, const void* k, const void* v,
                               zebra_seq kvs, const float* kbar, const float* vbar,
                               const int32_t* sel, int32_t q_tile, int32_t k_tile, int32_t top_k,
                               float scale, void* o, zebra_seq os, zebra_dtype o_dtype,
                               uint32_t flags, float* lse_out, void* workspace,
                               size_t workspace_bytes, void* stream) {
  zebra_status st;
  const uint32_t known = ZEBRA_SPARSE_NO_LANDMARKS | ZEBRA_SPARSE_LANDMARK_LOG_COUNT;
  if ((flags & ~known) != 0u || flags == known) return ZEBRA_ERR_INVALID_ARG;
  const bool landmarks = (flags & ZEBRA_SPARSE_NO_LANDMARKS) == 0u;
  if ((st = check_seq(q, qs, false)) != ZEBRA_OK) return st;
  if ((st = check_seq(k, kvs, false)) != ZEBRA_OK) return st;
  if ((st = check_seq(v, kvs, false)) != ZEBRA_OK) return st;
  if ((st = check_seq(o, os, true)) != ZEBRA_OK) return st;
  if (o_dtype != ZEBRA_BF16 && o_dtype != ZEBRA_F32) return ZEBRA_ERR_INVALID_ARG;
  if (qs.n_heads != kvs.n_heads || os.n_heads != qs.n_heads || os.n_tokens != qs.n_tokens)
    return ZEBRA_ERR_INVALID_ARG;
  if (q_tile != 32 && q_tile != 64 && q_tile != 128) return ZEBRA_ERR_UNSUPPORTED;
  if (k_tile != 32 && k_tile != 64) return ZEBRA_ERR_UNSUPPORTED;
  if (!(scale > 0.f) || scale > 1e30f) return ZEBRA_ERR_INVALID_ARG;
  if (seq_empty(qs)) return ZEBRA_OK;
  if (kvs.n_tokens == 0) return ZEBRA_ERR_INVALID_ARG;  // no keys to attend to
  const int64_t tk = ceil_div(kvs.n_tokens, k_tile);
  if (tk > kMaxKeyTiles) return ZEBRA_ERR_UNSUPPORTED;
  const int64_t tq = ceil_div(qs.n_tokens, q_tile);
  if (tq * qs.n_heads > (int64_t)UINT32_MAX) return ZEBRA_ERR_UNSUPPORTED;
  if (top_k < 1 || top_k > tk) return ZEBRA_ERR_INVALID_ARG;
  const bool dense = top_k == tk;
  const bool use_lm = !dense && landmarks;  // kbar and vbar are read
  if (!dense && sel == nullptr) return ZEBRA_ERR_INVALID_ARG;
  if (use_lm && (kbar == nullptr || vbar == nullptr)) return ZEBRA_ERR_INVALID_ARG;
  // the kernel addresses rows of one key tile with 32-bit byte offsets
  if (kvs.stride_token > (int64_t)1 << 24) return ZEBRA_ERR_UNSUPPORTED;
  const size_t need = zebra::sparse_workspace_bytes(qs.n_tokens, kvs.n_tokens, kvs.n_heads,
                                                    q_tile, k_tile, top_k);
  if (workspace == nullptr || workspace_bytes < need) return ZEBRA_ERR_WORKSPACE;
  if (((uintptr_t)workspace % 16) != 0) return ZEBRA_ERR_INVALID_ARG;
  if (use_lm && (((uintptr_t)kbar % 16) != 0 || ((uintptr_t)vbar % 16) != 0))
    return ZEBRA_ERR_INVALID_ARG;
  if (!dense && ((uintptr_t)sel % 4) != 0) return ZEBRA_ERR_INVALID_ARG;
  const size_t oel = o_dtype == ZEBRA_F32 ? 4 : 2;
  if (o_dtype == ZEBRA_F32 && (os.stride_token % 8 != 0 || os.stride_head % 8 != 0))
    return ZEBRA_ERR_UNSUPPORTED;
  const Range orng = seq_range(o, os, oel);
  std::vector<Range> inputs = {seq_range(q, qs, 2), seq_range(k, kvs, 2), seq_range(v, kvs, 2)};
  if (use_lm) {
    inputs.push_back(flat_range(kbar, (uint64_t)kvs.n_heads * tk * zebra::kHeadDim, 4));
    inputs.push_back(flat_range(vbar, (uint64_t)kvs.n_heads * tk * zebra::kHeadDim, 4));
  }
  if (!dense) inputs.push_back(flat_range(sel, (uint64_t)kvs.n_heads * tq * top_k, 4));
  const Range ws = flat_range(workspace, need, 1);
  if (overlaps(ws, orng)) return ZEBRA_ERR_INVALID_ARG;
  for (const Range& r : inputs)
    if (overlaps(ws, r)) return ZEBRA_ERR_INVALID_ARG;
  for (const Range& r : inputs)
    if (overlaps(orng, r)) return ZEBRA_ERR_INVALID_ARG;
  if (lse_out != nullptr) {
    if (((uintptr_t)lse_out % 4) != 0) return ZEBRA_ERR_INVALID_ARG;
    const Range lr = flat_range(lse_out, (uint64_t)qs.n_heads * qs.n_tokens, 4);
    if (overlaps(lr, orng) || overlaps(lr, ws)) return ZEBRA_ERR_INVALID_ARG;
    for (const Range& r : inputs)
      if (overlaps(lr, r)) return ZEBRA_ERR_INVALID_ARG;
  }
  return hip_status(zebra::launch_tile_sparse(
      (const uint16_t*)q, qs.n_tokens, qs.stride_token, qs.stride_head, (const uint16_t*)k,
      (const uint16_t*)v, kvs.n_tokens, kvs.stride_token, kvs.stride_head, qs.n_heads,
      use_lm ? kbar : nullptr, use_lm ? vbar : nullptr, dense ? nullptr : sel, q_tile, k_tile,
      top_k, scale, o, os.stride_token, os.stride_head, o_dtype == ZEBRA_F32,
      dense ? 0u : flags, workspace, (hipStream_t)stream, lse_out));
}

zebra_status zebra_tile_sparse_attn_ex(const void* q, zebra_seq qs, const void* k, const void* v,
                                       zebra_seq kvs, const float* kbar, const float* vbar,
                                       const int32_t* sel, int32_t q_tile, int32_t k_tile,
                                       int32_t top_k, float scale, void* o, zebra_seq os,
                                       zebra_dtype o_dtype, uint32_t flags, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  return sparse_fwd(q, qs, k, v, kvs, kbar, vbar, sel, q_tile, k_tile, top_k, scale, o, os,
                    o_dtype, flags, nullptr, workspace, workspace_bytes, stream);
}

zebra_status zebra_tile_sparse_attn_lse(const void* q, zebra_seq qs, const void* k, const void* v,
                                        zebra_seq kvs, const float* kbar, const float* vbar,
                                        const int32_t* sel, int32_t q_tile, int32_t k_tile,
                                        int32_t top_k, float scale, void* o, zebra_seq os,
                                        zebra_dtype o_dtype, uint32_t flags, float* lse_out,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  if (lse_out == nullptr && !seq_empty(qs)) return ZEBRA_ERR_INVALID_ARG;
  return sparse_fwd(q, qs, k, v, kvs, kbar, vbar, sel, q_tile, k_tile, top_k, scale, o, os,
                    o_dtype, flags, lse_out, workspace, workspace_bytes, stream);
}

size_t zebra_block_mass_workspace(int64_t n_q, int32_t n_heads) {
  if (n_q < 0 || n_heads < 0) return 0;
  return zebra::mass_workspace_bytes(n_q, n_heads);
}

zebra_status zebra_block_mass(const void* q, zebra_seq qs, const void* k, zebra_seq ks,
                              int32_t q_tile, int32_t k_tile, float scale, float* mass_out,
                              void* workspace, size_t workspace_bytes, void* stream) {
  zebra_status st;
  if ((st = check_seq(q, qs, false)) != ZEBRA_OK) return st;
  if ((st = check_seq(k, ks, false)) != ZEBRA_OK) return st;
  if (qs.n_heads != ks.n_heads) return ZEBRA_ERR_INVALID_ARG;
  if (q_tile != 32 && q_tile != 64 && q_tile != 128) return ZEBRA_ERR_UNSUPPORTED;
  if (k_tile != 32 && k_tile != 64) return ZEBRA_ERR_UNSUPPORTED;
  if (!(scale > 0.f) || scale > 1e30f) return ZEBRA_ERR_INVALID_ARG;
  if (seq_empty(qs)) return ZEBRA_OK;
  if (ks.n_tokens == 0) return ZEBRA_ERR_INVALID_ARG;
  const int64_t tk = ceil_div(ks.n_tokens, k_tile);
  if (tk > kMaxKeyTiles) return ZEBRA_ERR_UNSUPPORTED;
  const int64_t tq = ceil_div(qs.n_tokens, q_tile);
  if (tq > (int64_t)INT32_MAX) return ZEBRA_ERR_UNSUPPORTED;
  if (mass_out == nullptr || ((uintptr_t)mass_out % 4) != 0) return ZEBRA_ERR_INVALID_ARG;
  const size_t need = zebra::mass_workspace_bytes(qs.n_tokens, qs.n_heads);
  if (workspace == nullptr || workspace_bytes < need) return ZEBRA_ERR_WORKSPACE;
  if (((uintptr_t)workspace % 16) != 0) return ZEBRA_ERR_INVALID_ARG;
  const Range out = flat_range(mass_out, (uint64_t)qs.n_heads * tq * tk, 4);
  const Range ws = flat_range(workspace, need, 1);
  for (const Range& r : {seq_range(q, qs, 2), seq_range(k, ks, 2)})
    if (overlaps(out, r) || overlaps(ws, r)) return ZEBRA_ERR_INVALID_ARG;
  if (overlaps(out, ws)) return ZEBRA_ERR_INVALID_ARG;
  return hip_status(zebra::launch_block_mass(
      (const uint16_t*)q, qs.n_tokens, qs.stride_token, qs.stride_head, (const uint16_t*)k,
      ks.n_tokens, ks.stride_token, ks.stride_head, qs.n_heads, q_tile, k_tile, scale,
      mass_out, workspace, (hipStream_t)stream));
}

size_t zebra_linear_attn_workspace(int64_t n_kv, int32_t n_heads, int32_t head_dim) {
  if (n_kv < 0 || n_heads <= 0 || head_dim != zebra::kHeadDim) return 0;
  return zebra::linear_workspace_bytes(n_kv, n_heads);
}

zebra_status zebra_linear_attn(const void* q, zebra_seq qs, const void* k, const void* v,
                               zebra_seq kvs, const float* aff_scale, const float* aff_bias,
                               void* o, zebra_seq os, zebra_dtype o_dtype, void* workspace,
                               size_t workspace_bytes, void* stream) {
  zebra_status st;
  if ((st = check_seq(q, qs, false)) != ZEBRA_OK) return st;
  if ((st = check_seq(k, kvs, false)) != ZEBRA_OK) return st;
  if ((st = check_seq(v, kvs, false)) != ZEBRA_OK) return st;
  if ((st = check_seq(o, os, true)) != ZEBRA_OK) return st;
  if (o_dtype != ZEBRA_BF16 && o_dtype != ZEBRA_F32) return ZEBRA_ERR_INVALID_ARG;
  if (qs.n_heads != kvs.n_heads || os.n_heads != qs.n_heads || os.n_tokens != qs.n_tokens)
    return ZEBRA_ERR_INVALID_ARG;
  if (seq_empty(qs)) return ZEBRA_OK;
  if (kvs.n_tokens == 0) return ZEBRA_ERR_INVALID_ARG;  // the normaliser would be zero
  const size_t need = zebra::linear_workspace_bytes(kvs.n_tokens, kvs.n_heads);
  if (workspace == nullptr || workspace_bytes < need) return ZEBRA_ERR_WORKSPACE;
  if (((uintptr_t)workspace % 16) != 0) return ZEBRA_ERR_INVALID_ARG;
  if (((uintptr_t)aff_scale % 4) != 0 || ((uintptr_t)aff_bias % 4) != 0)
    return ZEBRA_ERR_INVALID_ARG;
  if (o_dtype == ZEBRA_F32 && (os.stride_token % 8 != 0 || os.stride_head % 8 != 0))
    return ZEBRA_ERR_UNSUPPORTED;
  const size_t oel = o_dtype == ZEBRA_F32 ? 4 : 2;
  const Range orng = seq_range(o, os, oel);
  const Range ws = flat_range(workspace, need, 1);
  const uint64_t aff_n = (uint64_t)qs.n_heads * zebra::kHeadDim;
  const Range inputs[] = {seq_range(q, qs, 2), seq_range(k, kvs, 2), seq_range(v, kvs, 2),
                          flat_range(aff_scale, aff_n, 4), flat_range(aff_bias, aff_n, 4)};
  if (overlaps(ws, orng)) return ZEBRA_ERR_INVALID_ARG;
  for (const Range& r : inputs)
    if (overlaps(orng, r) || overlaps(ws, r)) return ZEBRA_ERR_INVALID_ARG;
  return hip_status(zebra::launch_linear(
      (const uint16_t*)q, qs.n_tokens, qs.stride_token, qs.stride_head, (const uint16_t*)k,
      (const uint16_t*)v, kvs.n_tokens, kvs.stride_token, kvs.stride_head, qs.n_heads,
      aff_scale, aff_bias, o, os.stride_token, os.stride_head, o_dtype == ZEBRA_F32, workspace,
      (hipStream_t)stream));
}

size_t zebra_linear_attn_noalloc_max_bytes(void) { return zebra::kNoAllocScratchBytes; }

zebra_status zebra_linear_attn_noalloc(const void* q, zebra_seq qs, const void* k, const void* v,
                                       zebra_seq kvs, const float* aff_scale,
                                       const float* aff_bias, void* o, zebra_seq os,
                                       zebra_dtype o_dtype, void* stream) {
  zebra_status st;
  if ((st = check_seq(q, qs, false)) != ZEBRA_OK) return st;
  if ((st = check_seq(k, kvs, false)) != ZEBRA_OK) return st;
  if ((st = check_seq(v, kvs, false)) != ZEBRA_OK) return st;
  if ((st = check_seq(o, os, true)) != ZEBRA_OK) return st;
  if (o_dtype != ZEBRA_BF16 && o_dtype != ZEBRA_F32) return ZEBRA_ERR_INVALID_ARG;
  if (qs.n_heads != kvs.n_heads || os.n_heads != qs.n_heads || os.n_tokens != qs.n_tokens)
    return ZEBRA_ERR_INVALID_ARG;
  if (seq_empty(qs)) return ZEBRA_OK;
  if (kvs.n_tokens == 0) return ZEBRA_ERR_INVALID_ARG;
  const size_t need = zebra::linear_workspace_bytes(kvs.n_tokens, kvs.n_heads);
  if (need > zebra::kNoAllocScratchBytes) return ZEBRA_ERR_WORKSPACE;  // too many heads
  if (((uintptr_t)aff_scale % 4) != 0 || ((uintptr_t)aff_bias % 4) != 0)
    return ZEBRA_ERR_INVALID_ARG;
  if (o_dtype == ZEBRA_F32 && (os.stride_token % 8 != 0 || os.stride_head % 8 != 0))
    return ZEBRA_ERR_UNSUPPORTED;
  const Range orng = seq_range(o, os, o_dtype == ZEBRA_F32 ? 4 : 2);
  const uint64_t aff_n = (uint64_t)qs.n_heads * zebra::kHeadDim;
  const Range inputs[] = {seq_range(q, qs, 2), seq_range(k, kvs, 2), seq_range(v, kvs, 2),
                          flat_range(aff_scale, aff_n, 4), flat_range(aff_bias, aff_n, 4)};
  for (const Range& r : inputs)
    if (overlaps(orng, r)) return ZEBRA_ERR_INVALID_ARG;
  void* scratch = nullptr;
  if (zebra::noalloc_scratch(&scratch) != hipSuccess) return ZEBRA_ERR_HIP;
  return hip_status(zebra::launch_linear(
      (const uint16_t*)q, qs.n_tokens, qs.stride_token, qs.stride_head, (const uint16_t*)k,
      (const uint16_t*)v, kvs.n_tokens, kvs.stride_token, kvs.stride_head, qs.n_heads,
      aff_scale, aff_bias, o, os.stride_token, os.stride_head, o_dtype == ZEBRA_F32, scratch,
      (hipStream_t)stream));
}

namespace {

zebra_status fit_common(const float* x, const float* y, int32_t m, int32_t n_heads,
                        int32_t head_dim, float* scale_out, float* bias_out,
                        int32_t* n_degenerate_out, bool centred, void* stream) {
  if (m < 1 || n_heads < 0) return ZEBRA_ERR_INVALID_ARG;
  if (head_dim != zebra::kHeadDim) return ZEBRA_ERR_UNSUPPORTED;
  if (x == nullptr || y == nullptr || scale_out == nullptr || bias_out == nullptr)
    return ZEBRA_ERR_INVALID_ARG;
  if (((uintptr_t)x % 4) != 0 || ((uintptr_t)y % 4) != 0 || ((uintptr_t)scale_out % 4) != 0 ||
      ((uintptr_t)bias_out % 4) != 0 || ((uintptr_t)n_degenerate_out % 4) != 0)
    return ZEBRA_ERR_INVALID_ARG;
  const uint64_t nin = (uint64_t)n_heads * m * head_dim, nout = (uint64_t)n_heads * head_dim;
  const Range xr = flat_range(x, nin, 4), yr = flat_range(y, nin, 4);
  const Range ar = flat_range(scale_out, nout, 4), br = flat_range(bias_out, nout, 4);
  const Range dr = flat_range(n_degenerate_out, 1, 4);
  const Range outs[] = {ar, br, dr};
  for (const Range& o : outs)
    if (overlaps(o, xr) || overlaps(o, yr)) return ZEBRA_ERR_INVALID_ARG;
  if (overlaps(ar, br) || overlaps(ar, dr) || overlaps(br, dr)) return ZEBRA_ERR_INVALID_ARG;
  return hip_status(zebra::launch_fit(x, y, m, n_heads, scale_out, bias_out, n_degenerate_out,
                                      centred, (hipStream_t)stream));
}

}  // namespace

zebra_status zebra_fit_affine(const float* x, const float* y, int32_t m, int32_t n_heads,
                              int32_t head_dim, float* scale_out, float* bias_out,
                              int32_t* n_degenerate_out, void* stream) {
  return fit_common(x, y, m, n_heads, head_dim, scale_out, bias_out, n_degenerate_out, true,
                    stream);
}

zebra_status zebra_fit_scale_only(const float* x, const float* y, int32_t m, int32_t n_heads,
                                  int32_t head_dim, float* scale_out, float* bias_out,
                                  int32_t* n_degenerate_out, void* stream) {
  return fit_common(x, y, m, n_heads, head_dim, scale_out, bias_out, n_degenerate_out, false,
                    stream);
}

size_t zebra_tile_sparse_attn_backward_workspace(int64_t n_q, int64_t n_kv, int32_t n_heads,
                                                 int32_t head_dim, int32_t q_tile, int32_t k_tile,
                                                 int32_t top_k) {
  if (n_q < 0 || n_kv < 1 || n_heads <= 0 || head_dim != zebra::kHeadDim) return 0;
  if (q_tile != 32 && q_tile != 64 && q_tile != 128) return 0;
  if (k_tile != 32 && k_tile != 64) return 0;
  const int64_t tk = ceil_div(n_kv, k_tile);
  if (top_k < 1 || top_k > tk) return 0;
  return zebra::sparse_bwd_workspace_bytes(n_q, n_kv, n_heads, q_tile, k_tile, top_k);
}

// zebra_tile_sparse_attn_backward, _backward_lse and _backward_saved: lse_in (float32
// [H][Nq], from zebra_tile_sparse_attn_lse with the same arguments) or NULL; out_in (that
// call's float32 output, layout os) or NULL
static zebra_status sparse_bwd(
    const void* q, zebra_seq qs, const void* k, const void* v, zebra_seq kvs, const float* kbar,
    const float* vbar, const int32_t* sel, int32_t q_tile, int32_t k_tile, int32_t top_k,
    float scale, uint32_t flags, const float* lse_in, const float* out_in, zebra_seq os,
    const void* dout, zebra_seq dos, zebra_dtype g_dtype, void* dq, zebra_seq dqs, void* dk,
    void* dv, zebra_seq dkvs, void* workspace, size_t workspace_bytes, void* stream) {
  zebra_status st;
  const uint32_t known = ZEBRA_SPARSE_NO_LANDMARKS | ZEBRA_SPARSE_LANDMARK_LOG_COUNT;
  if ((flags & ~known) != 0u || flags == known) return ZEBRA_ERR_INVALID_ARG;
  if ((st = check_seq(q, qs, false)) != ZEBRA_OK) return st;
  if ((st = check_seq(k, kvs, false)) != ZEBRA_OK) return st;
  if ((st = check_seq(v, kvs, false)) != ZEBRA_OK) return st;
  if ((st = check_seq(dout, dos, false)) != ZEBRA_OK) return st;
  if ((st = check_seq(dq, dqs, true)) != ZEBRA_OK) return st;
  if ((st = check_seq(dk, dkvs, true)) != ZEBRA_OK) return st;
  if ((st = check_seq(dv, dkvs, true)) != ZEBRA_OK) return st;
  if (g_dtype != ZEBRA_BF16 && g_dtype != ZEBRA_F32) return ZEBRA_ERR_INVALID_ARG;
  const int32_t h = qs.n_heads;
  if (kvs.n_heads != h || dos.n_heads != h || dqs.n_heads != h || dkvs.n_heads != h ||
      dos.n_tokens != qs.n_tokens || dqs.n_tokens != qs.n_tokens ||
      dkvs.n_tokens != kvs.n_tokens)
    return ZEBRA_ERR_INVALID_ARG;
  if (q_tile != 32 && q_tile != 64 && q_tile != 128) return ZEBRA_ERR_UNSUPPORTED;
  if (k_tile != 32 && k_tile != 64) return ZEBRA_ERR_UNSUPPORTED;
  if (!(scale > 0.f) || scale > 1e30f) return ZEBRA_ERR_INVALID_ARG;
  if (kvs.n_tokens == 0) return ZEBRA_ERR_INVALID_ARG;
  const int64_t tk = ceil_div(kvs.n_tokens, k_tile);
  if (tk > kMaxKeyTiles) return ZEBRA_ERR_UNSUPPORTED;
  const int64_t tq = ceil_div(qs.n_tokens, q_tile);
  if (tq * h > (int64_t)INT32_MAX || tq * top_k > (int64_t)INT32_MAX / (h > 0 ? h : 1))
    return ZEBRA_ERR_UNSUPPORTED;
  if (top_k < 1 || top_k > tk) return ZEBRA_ERR_INVALID_ARG;
  if (sel == nullptr || ((uintptr_t)sel % 4) != 0) return ZEBRA_ERR_INVALID_ARG;
  const bool use_lm = top_k < tk && (flags & ZEBRA_SPARSE_NO_LANDMARKS) == 0u;
  if (use_lm && (kbar == nullptr || vbar == nullptr || ((uintptr_t)kbar % 16) != 0 ||
                 ((uintptr_t)vbar % 16) != 0))
    return ZEBRA_ERR_INVALID_ARG;
  if (kvs.stride_token > (int64_t)1 << 24) return ZEBRA_ERR_UNSUPPORTED;
  const size_t gel = g_dtype == ZEBRA_F32 ? 4 : 2;
  if (g_dtype == ZEBRA_F32) {
    for (const zebra_seq* g : {&dos, &dqs, &dkvs})
      if (g->stride_token % 8 != 0 || g->stride_head % 8 != 0) return ZEBRA_ERR_UNSUPPORTED;
  }
  const size_t need = zebra::sparse_bwd_workspace_bytes(qs.n_tokens, kvs.n_tokens, h, q_tile,
                                                        k_tile, top_k);
  if (workspace == nullptr || workspace_bytes < need) return ZEBRA_ERR_WORKSPACE;
  if (((uintptr_t)workspace % 16) != 0) return ZEBRA_ERR_INVALID_ARG;
  std::vector<Range> ins = {seq_range(q, qs, 2), seq_range(k, kvs, 2), seq_range(v, kvs, 2),
                            seq_range(dout, dos, gel),
                            flat_range(sel, (uint64_t)h * tq * top_k, 4)};
  if (use_lm) {
    ins.push_back(flat_range(kbar, (uint64_t)h * tk * zebra::kHeadDim, 4));
    ins.push_back(flat_range(vbar, (uint64_t)h * tk * zebra::kHeadDim, 4));
  }
  if (lse_in != nullptr) {
    if (((uintptr_t)lse_in % 4) != 0) return ZEBRA_ERR_INVALID_ARG;
    ins.push_back(flat_range(lse_in, (uint64_t)h * qs.n_tokens, 4));
  }
  if (out_in != nullptr) {  // float32, read as 16-byte vectors
    if ((st = check_seq(out_in, os, false)) != ZEBRA_OK) return st;
    if (os.n_heads != h || os.n_tokens != qs.n_tokens) return ZEBRA_ERR_INVALID_ARG;
    ins.push_back(seq_range(out_in, os, 4));
  }
  const Range outs[] = {seq_range(dq, dqs, gel), seq_range(dk, dkvs, gel),
                        seq_range(dv, dkvs, gel), flat_range(workspace, need, 1)};
  for (size_t i = 0; i < 4; ++i) {
    for (const Range& r : ins)
      if (overlaps(outs[i], r)) return ZEBRA_ERR_INVALID_ARG;
    for (size_t j = i + 1; j < 4; ++j)
      if (overlaps(outs[i], outs[j])) return ZEBRA_ERR_INVALID_ARG;
  }
  return hip_status(zebra::launch_tile_sparse_bwd(
      (const uint16_t*)q, qs.n_tokens, qs.stride_token, qs.stride_head, (const uint16_t*)k,
      (const uint16_t*)v, kvs.n_tokens, kvs.stride_token, kvs.stride_head, h,
      use_lm ? kbar : nullptr, use_lm ? vbar : nullptr, sel, q_tile, k_tile, top_k, scale,
      top_k < tk ? flags : 0u, dout, dos.stride_token, dos.stride_head, g_dtype == ZEBRA_F32, dq,
      dqs.stride_token, dqs.stride_head, dk, dv, dkvs.stride_token, dkvs.stride_head, workspace,
      (hipStream_t)stream, lse_in, out_in, os.stride_token, os.stride_head));
}

zebra_status zebra_tile_sparse_attn_backward(
    const void* q, zebra_seq qs, const void* k, const void* v, zebra_seq kvs, const float* kbar,
    const float* vbar, const int32_t* sel, int32_t q_tile, int32_t k_tile, int32_t top_k,
    float scale, uint32_t flags, const void* dout, zebra_seq dos, zebra_dtype g_dtype, void* dq,
    zebra_seq dqs, void* dk, void* dv, zebra_seq dkvs, void* workspace, size_t workspace_bytes,
    void* stream) {
  return sparse_bwd(q, qs, k, v, kvs, kbar, vbar, sel, q_tile, k_tile, top_k, scale, flags,
                    nullptr, nullptr, zebra_seq{}, dout, dos, g_dtype, dq, dqs, dk, dv, dkvs,
                    workspace, workspace_bytes, stream);
}

zebra_status zebra_tile_sparse_attn_backward_lse(
    const void* q, zebra_seq qs, const void* k, const void* v, zebra_seq kvs, const float* kbar,
    const float* vbar, const int32_t* sel, int32_t q_tile, int32_t k_tile, int32_t top_k,
    float scale, uint32_t flags, const float* lse, const void* dout, zebra_seq dos,
    zebra_dtype g_dtype, void* dq, zebra_seq dqs, void* dk, void* dv, zebra_seq dkvs,
    void* workspace, size_t workspace_bytes, void* stream) {
  if (lse == nullptr && !seq_empty(qs)) return ZEBRA_ERR_INVALID_ARG;
  return sparse_bwd(q, qs, k, v, kvs, kbar, vbar, sel, q_tile, k_tile, top_k, scale, flags, lse,
                    nullptr, zebra_seq{}, dout, dos, g_dtype, dq, dqs, dk, dv, dkvs, workspace,
                    workspace_bytes, stream);
}

zebra_status zebra_tile_sparse_attn_backward_saved(
    const void* q, zebra_seq qs, const void* k, const void* v, zebra_seq kvs, const float* kbar,
    const float* vbar, const int32_t* sel, int32_t q_tile, int32_t k_tile, int32_t top_k,
    float scale, uint32_t flags, const float* lse, const float* out, zebra_seq os,
    const void* dout, zebra_seq dos, zebra_dtype g_dtype, void* dq, zebra_seq dqs, void* dk,
    void* dv, zebra_seq dkvs, void* workspace, size_t workspace_bytes, void* stream) {
  if ((lse == nullptr || out == nullptr) && !seq_empty(qs)) return ZEBRA_ERR_INVALID_ARG;
  if (seq_empty(qs)) out = nullptr;
  return sparse_bwd(q, qs, k, v, kvs, kbar, vbar, sel, q_tile, k_tile, top_k, scale, flags, lse,
                    out, os, dout, dos, g_dtype, dq, dqs, dk, dv, dkvs, workspace,
                    workspace_bytes, stream);
}

size_t zebra_linear_attn_backward_workspace(int64_t n_q, int64_t n_kv, int32_t n_heads,
                                            int32_t head_dim) {
  if (n_q < 0 || n_kv < 0 || n_heads <= 0 || head_dim != zebra::kHeadDim) return 0;
  return zebra::linear_bwd_workspace_bytes(n_q, n_kv, n_heads);
}

zebra_status zebra_linear_attn_backward(const void* q, zebra_seq qs, const void* k, const void* v,
                                        zebra_seq kvs, const float* aff_scale, const void* dout,
                                        zebra_seq dos, zebra_dtype g_dtype, void* dq,
                                        zebra_seq dqs, void* dk, void* dv, zebra_seq dkvs,
                                        float* d_scale, float* d_bias, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  zebra_status st;
  if ((st = check_seq(q, qs, false)) != ZEBRA_OK) return st;
  if ((st = check_seq(k, kvs, false)) != ZEBRA_OK) return st;
  if ((st = check_seq(v, kvs, false)) != ZEBRA_OK) return st;
  if ((st = check_seq(dout, dos, false)) != ZEBRA_OK) return st;
  if ((st = check_seq(dq, dqs, true)) != ZEBRA_OK) return st;
  if ((st = check_seq(dk, dkvs, true)) != ZEBRA_OK) return st;
  if ((st = check_seq(dv, dkvs, true)) != ZEBRA_OK) return st;
  if (g_dtype != ZEBRA_BF16 && g_dtype != ZEBRA_F32) return ZEBRA_ERR_INVALID_ARG;
  const int32_t h = qs.n_heads;
  if (kvs.n_heads != h || dos.n_heads != h || dqs.n_heads != h || dkvs.n_heads != h ||
      dos.n_tokens != qs.n_tokens || dqs.n_tokens != qs.n_tokens ||
      dkvs.n_tokens != kvs.n_tokens)
    return ZEBRA_ERR_INVALID_ARG;
  if (seq_empty(qs) && seq_empty(kvs)) return ZEBRA_OK;
  if (kvs.n_tokens == 0) return ZEBRA_ERR_INVALID_ARG;  // the normaliser would be zero
  const size_t need = zebra::linear_bwd_workspace_bytes(qs.n_tokens, kvs.n_tokens, h);
  if (workspace == nullptr || workspace_bytes < need) return ZEBRA_ERR_WORKSPACE;
  if (((uintptr_t)workspace % 16) != 0) return ZEBRA_ERR_INVALID_ARG;
  if (((uintptr_t)aff_scale % 4) != 0 || ((uintptr_t)d_scale % 4) != 0 ||
      ((uintptr_t)d_bias % 4) != 0)
    return ZEBRA_ERR_INVALID_ARG;
  const size_t gel = g_dtype == ZEBRA_F32 ? 4 : 2;
  if (g_dtype == ZEBRA_F32) {
    for (const zebra_seq* g : {&dos, &dqs, &dkvs})
      if (g->stride_token % 8 != 0 || g->stride_head % 8 != 0) return ZEBRA_ERR_UNSUPPORTED;
  }
  const uint64_t hn = (uint64_t)h * zebra::kHeadDim;
  const Range outs[] = {seq_range(dq, dqs, gel), seq_range(dk, dkvs, gel),
                        seq_range(dv, dkvs, gel), flat_range(d_scale, hn, 4),
                        flat_range(d_bias, hn, 4), flat_range(workspace, need, 1)};
  const Range ins[] = {seq_range(q, qs, 2), seq_range(k, kvs, 2), seq_range(v, kvs, 2),
                       seq_range(dout, dos, gel), flat_range(aff_scale, hn, 4)};
  for (size_t i = 0; i < 6; ++i) {
    for (const Range& r : ins)
      if (overlaps(outs[i], r)) return ZEBRA_ERR_INVALID_ARG;
    for (size_t j = i + 1; j < 6; ++j)
      if (overlaps(outs[i], outs[j])) return ZEBRA_ERR_INVALID_ARG;
  }
  return hip_status(zebra::launch_linear_bwd(
      (const uint16_t*)q, qs.n_tokens, qs.stride_token, qs.stride_head, (const uint16_t*)k,
      (const uint16_t*)v, kvs.n_tokens, kvs.stride_token, kvs.stride_head, h, aff_scale, dout,
      dos.stride_token, dos.stride_head, dq, dqs.stride_token, dqs.stride_head, dk, dv,
      dkvs.stride_token, dkvs.stride_head, g_dtype == ZEBRA_F32, d_scale, d_bias, workspace,
      (hipStream_t)stream));
}

zebra_status zebra_spatial_order(int32_t n_views, int32_t n_special, int32_t grid_h,
                                 int32_t grid_w, int32_t block, int32_t* order_out,
                                 int64_t order_len) {
  if (n_views < 0 || n_special < 0 || grid_h < 0 || grid_w < 0 || block < 1)
    return ZEBRA_ERR_INVALID_ARG;
  const int64_t n = (int64_t)n_views * ((int64_t)n_special + (int64_t)grid_h * grid_w);
  if (n > (int64_t)INT32_MAX) return ZEBRA_ERR_UNSUPPORTED;
  if (order_len != n || (n > 0 && order_out == nullptr)) return ZEBRA_ERR_INVALID_ARG;
  zebra::spatial_order(n_views, n_special, grid_h, grid_w, block, order_out);
  return ZEBRA_OK;
}

zebra_status zebra_permute_tokens(const void* src, zebra_seq ss, const int32_t* order,
                                  int32_t inverse, zebra_dtype dtype, void* dst, zebra_seq ds,
                                  void* stream) {
  zebra_status st;
  if ((st = check_seq(src, ss, false)) != ZEBRA_OK) return st;
  if ((st = check_seq(dst, ds, true)) != ZEBRA_OK) return st;
  if (dtype != ZEBRA_BF16 && dtype != ZEBRA_F32) return ZEBRA_ERR_INVALID_ARG;
  if (inverse != 0 && inverse != 1) return ZEBRA_ERR_INVALID_ARG;
  if (ss.n_heads != ds.n_heads || ss.n_tokens != ds.n_tokens) return ZEBRA_ERR_INVALID_ARG;
  if (seq_empty(ss)) return ZEBRA_OK;
  if (ss.n_tokens > (int64_t)INT32_MAX) return ZEBRA_ERR_UNSUPPORTED;
  if (order == nullptr || ((uintptr_t)order % 4) != 0) return ZEBRA_ERR_INVALID_ARG;
  const size_t el = dtype == ZEBRA_F32 ? 4 : 2;
  const Range sr = seq_range(src, ss, el), dr = seq_range(dst, ds, el);
  const Range orr = flat_range(order, (uint64_t)ss.n_tokens, 4);
  if (overlaps(dr, sr) || overlaps(dr, orr)) return ZEBRA_ERR_INVALID_ARG;
  return hip_status(zebra::launch_permute(src, ss.stride_token, ss.stride_head, dst,
                                          ds.stride_token, ds.stride_head, order, ss.n_tokens,
                                          ss.n_heads, (int32_t)el, inverse == 1,
                                          (hipStream_t)stream));
}

}  // extern "C"
