// Closed-form affine fit of the linear-attention output (gfx950).
//
// news.hamidun.com article ("Zebra3D speeds up 3D reconstruction..."), section
// "How Zebra3D works": the linear components are fitted by a closed-form
// affine transformation, no gradient descent. Per (head, channel), over m
// samples: a = sum (x - xbar)(y - ybar) / sum (x - xbar)^2, b = ybar - a xbar
// (centred normal equations; Zebra3D paper page, Table 3(a) contrasts this
// with an uncentred fit). A channel with sum (x - xbar)^2 <= 1e-30 m gets
// a = 0, b = ybar.
//
// Uncentered variant (Zebra3D paper page, Table 3(a), "Linear, uncentered
// fit"): the least-squares map through the origin, a = sum x y / sum x^2,
// b = 0, i.e. the same sums with the means taken as zero. A channel with
// sum x^2 <= 1e-30 m gets a = 0.
//
// One workgroup per head: 64 channels x 4 sample groups, float64 sums, the
// 4 groups combined in a fixed order (deterministic). Two passes: means, then
// centred sums (the uncentered fit skips the first).
#include "common.h"

namespace zebra {

namespace {

__global__ void zero_counter_kernel(int32_t* c) { *c = 0; }

__global__ __launch_bounds__(256) void fit_kernel(const float* __restrict__ x,
                                                  const float* __restrict__ y, int32_t m,
                                                  float* __restrict__ a_out,
                                                  float* __restrict__ b_out,
                                                  int32_t* __restrict__ n_deg,
                                                  int32_t centred) {
  __shared__ double red[2][4][kHeadDim];
  __shared__ int deg_count;
  const int h = blockIdx.x, c = threadIdx.x % kHeadDim, g = threadIdx.x / kHeadDim;
  const float* xh = x + (int64_t)h * m * kHeadDim;
  const float* yh = y + (int64_t)h * m * kHeadDim;
  if (threadIdx.x == 0) deg_count = 0;

  double xbar = 0.0, ybar = 0.0;
  if (centred) {
    double sx = 0.0, sy = 0.0;
    for (int i = g; i < m; i += 4) {
      sx += (double)xh[(int64_t)i * kHeadDim + c];
      sy += (double)yh[(int64_t)i * kHeadDim + c];
    }
    red[0][g][c] = sx;
    red[1][g][c] = sy;
    __syncthreads();
    xbar = (red[0][0][c] + red[0][1][c] + red[0][2][c] + red[0][3][c]) / m;
    ybar = (red[1][0][c] + red[1][1][c] + red[1][2][c] + red[1][3][c]) / m;
    __syncthreads();
  }

  double sxx = 0.0, sxy = 0.0;
  for (int i = g; i < m; i += 4) {
    const double dx = (double)xh[(int64_t)i * kHeadDim + c] - xbar;
    const double dy = (double)yh[(int64_t)i * kHeadDim + c] - ybar;
    sxx += dx * dx;
    sxy += dx * dy;
  }
  red[0][g][c] = sxx;
  red[1][g][c] = sxy;
  __syncthreads();
  if (g == 0) {
    const double txx = red[0][0][c] + red[0][1][c] + red[0][2][c] + red[0][3][c];
    const double txy = red[1][0][c] + red[1][1][c] + red[1][2][c] + red[1][3][c];
    const bool ok = txx > 1e-30 * (double)m;
    const double a = ok ? txy / txx : 0.0;
    a_out[h * kHeadDim + c] = (float)a;
    b_out[h * kHeadDim + c] = (float)(ybar - a * xbar);
    if (!ok) atomicAdd(&deg_count, 1);
  }
  __syncthreads();
  if (threadIdx.x == 0 && n_deg != nullptr && deg_count != 0) atomicAdd(n_deg, deg_count);
}

}  // namespace

hipError_t launch_fit(const float* x, const float* y, int32_t m, int32_t heads, float* a,
                      float* b, int32_t* n_deg, bool centred, hipStream_t s) {
  if (n_deg != nullptr) {
    hipLaunchKernelGGL(zero_counter_kernel, dim3(1), dim3(1), 0, s, n_deg);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (heads == 0) return hipSuccess;
  hipLaunchKernelGGL(fit_kernel, dim3(heads), dim3(256), 0, s, x, y, m, a, b, n_deg,
                     centred ? 1 : 0);
  return hipGetLastError();
}

}  // namespace zebra
