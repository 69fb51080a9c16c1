// Spatial tiles as a token permutation (gfx950).
//
// Zebra3D paper page: the sparse stages keep softmax over selected spatial
// tiles (abstract), and the appendix Tables 15-17 compare block-sparse with
// tile-sparse attention. Tiles here are contiguous runs of the token order,
// so spatial tiles come from putting the tokens in a spatial order first:
// per view, the special tokens, then the patch grid in s x s blocks taken in
// raster order of blocks, each block row-major (edge blocks are smaller).
// Attention is equivariant under a common permutation of queries and keys, so
// gather -> tile-sparse attention -> scatter gives the spatial-tile operator
// in the original order.
//
// permute_kernel moves 64-channel rows (bf16 or float32) by a device index
// vector: gather dst[h][i] = src[h][order[i]], or scatter dst[h][order[i]] =
// src[h][i]. Each thread moves one 16-byte piece of a row, so a row is one
// contiguous 128- or 256-byte access; it is an HBM copy, bound by bandwidth.
// Indices outside [0, n) move nothing.
#include <algorithm>

#include "common.h"

namespace zebra {

namespace {

__global__ __launch_bounds__(256) void permute_kernel(const uint8_t* __restrict__ src,
                                                      int64_t s_tok, int64_t s_head,
                                                      uint8_t* __restrict__ dst, int64_t d_tok,
                                                      int64_t d_head,
                                                      const int32_t* __restrict__ order,
                                                      int64_t n, int32_t heads, int32_t pieces,
                                                      int32_t scatter) {
  // strides in bytes; pieces = 16-byte pieces per row (8 for bf16, 16 for float32)
  const int64_t total = (int64_t)heads * n * pieces;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int piece = (int)(e % pieces);
    const int64_t row = e / pieces;
    const int64_t h = row / n, i = row - h * n;
    const int64_t j = order[i];
    if (j < 0 || j >= n) continue;
    const int64_t si = scatter ? i : j, di = scatter ? j : i;
    const u32x4 w = *(const u32x4*)(src + h * s_head + si * s_tok + 16 * piece);
    *(u32x4*)(dst + h * d_head + di * d_tok + 16 * piece) = w;
  }
}

}  // namespace

int64_t spatial_order(int32_t n_views, int32_t n_special, int32_t grid_h, int32_t grid_w,
                      int32_t block, int32_t* out) {
  const int64_t per_view = (int64_t)n_special + (int64_t)grid_h * grid_w;
  int64_t pos = 0;
  for (int32_t view = 0; view < n_views; ++view) {
    const int64_t base = view * per_view;
    for (int32_t t = 0; t < n_special; ++t) out[pos++] = (int32_t)(base + t);
    for (int32_t r0 = 0; r0 < grid_h; r0 += block)
      for (int32_t c0 = 0; c0 < grid_w; c0 += block)
        for (int32_t r = r0; r < grid_h && r < r0 + block; ++r)
          for (int32_t c = c0; c < grid_w && c < c0 + block; ++c)
            out[pos++] = (int32_t)(base + n_special + (int64_t)r * grid_w + c);
  }
  return pos;
}

hipError_t launch_permute(const void* src, int64_t s_tok, int64_t s_head, void* dst,
                          int64_t d_tok, int64_t d_head, const int32_t* order, int64_t n,
                          int32_t heads, int32_t elem_bytes, bool scatter, hipStream_t s) {
  if (n == 0 || heads == 0) return hipSuccess;
  const int32_t pieces = kHeadDim * elem_bytes / 16;
  const int64_t total = (int64_t)heads * n * pieces;
  const int64_t blocks = std::min<int64_t>((total + 255) / 256, (int64_t)1 << 20);
  hipLaunchKernelGGL(permute_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     (const uint8_t*)src, s_tok * elem_bytes, s_head * elem_bytes,
                     (uint8_t*)dst, d_tok * elem_bytes, d_head * elem_bytes, order, n, heads,
                     pieces, scatter ? 1 : 0);
  return hipGetLastError();
}

}  // namespace zebra
