// Tile pooling: mean key / mean value / mean query of every tile.
//
// Zebra3D paper page (thelatestinai.com), Figure 1 caption: omitted tiles are
// summarised by their mean key and mean value. The same means of the query
// tiles feed the tile scores.
//
// HBM-bound: each bf16 element is read once. One wave reduces one tile: lane
// l reads 16 bytes (channels 8*(l%8) .. +7) of token rows l/8, l/8 + 8, ...,
// so one wave-wide load covers 8 full 128-byte rows. Up to 8 loads per lane
// are issued before any arithmetic. The 8 row-partials are then combined
// with three xor-shuffles in a fixed order (deterministic).
#include "common.h"

namespace zebra {

namespace {

constexpr int kPoolWaves = 4;

__device__ __forceinline__ void add_row(float* acc, u32x4 w) {
  acc[0] += bf16lo(w.x);
  acc[1] += bf16hi(w.x);
  acc[2] += bf16lo(w.y);
  acc[3] += bf16hi(w.y);
  acc[4] += bf16lo(w.z);
  acc[5] += bf16hi(w.z);
  acc[6] += bf16lo(w.w);
  acc[7] += bf16hi(w.w);
}

__global__ __launch_bounds__(kPoolWaves * kWave) void pool_kernel(
    const uint16_t* __restrict__ x, int64_t n, int64_t st, int64_t sh, int32_t tile,
    int64_t n_tiles, float* __restrict__ out) {
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int64_t t = (int64_t)blockIdx.x * kPoolWaves + wave;
  const int h = blockIdx.y;
  if (t >= n_tiles) return;
  const int64_t s = t * tile;
  const int64_t e = min(n, s + (int64_t)tile);
  const int cg = lane & 7;
  const uint16_t* base = x + (int64_t)h * sh + 8 * cg;

  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int64_t tok = s + (lane >> 3);
  for (; tok + 56 < e; tok += 64) {
    u32x4 w[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) w[u] = *(const u32x4*)(base + (tok + 8 * u) * st);
#pragma unroll
    for (int u = 0; u < 8; ++u) add_row(acc, w[u]);
  }
  for (; tok < e; tok += 8) add_row(acc, *(const u32x4*)(base + tok * st));

#pragma unroll
  for (int o = 8; o < 64; o <<= 1) {
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] += __shfl_xor(acc[c], o, kWave);
  }
  if (lane < 8) {
    const float cnt = (float)(e - s);
    f32x4 lo = {acc[0] / cnt, acc[1] / cnt, acc[2] / cnt, acc[3] / cnt};
    f32x4 hi = {acc[4] / cnt, acc[5] / cnt, acc[6] / cnt, acc[7] / cnt};
    float* dst = out + ((int64_t)h * n_tiles + t) * kHeadDim + 8 * cg;
    *(f32x4*)dst = lo;
    *(f32x4*)(dst + 4) = hi;
  }
}

}  // namespace

hipError_t launch_pool(const uint16_t* x, int64_t n, int32_t heads, int64_t st, int64_t sh,
                       int32_t tile, float* out, hipStream_t s) {
  const int64_t n_tiles = (n + tile - 1) / tile;
  if (n_tiles == 0 || heads == 0) return hipSuccess;
  dim3 grid((unsigned)((n_tiles + kPoolWaves - 1) / kPoolWaves), (unsigned)heads);
  hipLaunchKernelGGL(pool_kernel, grid, dim3(kPoolWaves * kWave), 0, s, x, n, st, sh, tile,
                     n_tiles, out);
  return hipGetLastError();
}

}  // namespace zebra
