// Tile selection: pooled-query . pooled-key scores, then top-k per query tile.
//
// The tile-sparse stage computes only selected blocks (news.hamidun.com
// article "Zebra3D speeds up 3D reconstruction...", section "How Zebra3D
// works"). Score of query tile i and key tile j: s_ij = qbar_i . kbar_j in
// float32. Each (head, i) keeps the top_k key tiles under the order
// (s_ij descending, j ascending) and emits them in ascending order.
//
// Two kernels:
//  1. score_kernel: a K=64 float32 GEMM, 64x64 output tile per workgroup,
//     operands staged in LDS, sequential FMA over the 64 channels (the same
//     summation order for every element).
//  2. select_kernel: one workgroup per (head, query tile). The row's scores
//     sit in registers (contiguous index range per thread). The k-th largest
//     value tau is found exactly: min/max, a 2048-bin histogram on the value
//     range (a monotone binning, so equal scores share a bin), the bin where
//     the count from the top crosses k, then an exact rank among that bin's
//     members. Kept tiles are {s > tau} plus the lowest-indexed ties at tau,
//     written in index order through a block-wide scan. No sort, no float
//     atomics; the result does not depend on scheduling.
#include "common.h"

namespace zebra {

namespace {

constexpr int kScoreTile = 64;

__global__ __launch_bounds__(256) void score_kernel(const float* __restrict__ qbar,
                                                    const float* __restrict__ kbar, int32_t tq,
                                                    int32_t tk, float* __restrict__ scores) {
  __shared__ float qs[kScoreTile][kHeadDim + 1];
  __shared__ float ks[kScoreTile][kHeadDim + 1];
  const int h = blockIdx.z;
  const int i0 = blockIdx.y * kScoreTile;
  const int j0 = blockIdx.x * kScoreTile;
  const float* qh = qbar + (int64_t)h * tq * kHeadDim;
  const float* kh = kbar + (int64_t)h * tk * kHeadDim;
  for (int e = threadIdx.x; e < kScoreTile * kHeadDim; e += 256) {
    const int r = e / kHeadDim, c = e % kHeadDim;
    qs[r][c] = (i0 + r < tq) ? qh[(int64_t)(i0 + r) * kHeadDim + c] : 0.f;
    ks[r][c] = (j0 + r < tk) ? kh[(int64_t)(j0 + r) * kHeadDim + c] : 0.f;
  }
  __syncthreads();
  const int tx = threadIdx.x % 16;  // columns tx + 16 b
  const int ty = threadIdx.x / 16;  // rows 4 ty + a
  float acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.f;
  for (int c = 0; c < kHeadDim; ++c) {
    float qv[4], kv[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) qv[a] = qs[4 * ty + a][c];
#pragma unroll
    for (int b = 0; b < 4; ++b) kv[b] = ks[tx + 16 * b][c];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[a][b] = __builtin_fmaf(qv[a], kv[b], acc[a][b]);
  }
  float* out = scores + (int64_t)h * tq * tk;
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int i = i0 + 4 * ty + a;
    if (i >= tq) continue;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int j = j0 + tx + 16 * b;
      if (j < tk) out[(int64_t)i * tk + j] = acc[a][b];
    }
  }
}

constexpr int kBins = 2048;

// Inclusive prefix sum over the block (NT threads), integer.
template <int NT>
__device__ __forceinline__ uint32_t block_inclusive_scan(uint32_t v, uint32_t* wave_tot) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const uint32_t u = __shfl_up(v, o, kWave);
    if (lane >= o) v += u;
  }
  if (lane == kWave - 1) wave_tot[wave] = v;
  __syncthreads();
  uint32_t before = 0;
  for (int w = 0; w < wave; ++w) before += wave_tot[w];
  __syncthreads();
  return v + before;
}

template <int NT>
__device__ __forceinline__ float block_reduce_max(float v, float* tmp) {
  v = wave_max(v);
  if (threadIdx.x % kWave == 0) tmp[threadIdx.x / kWave] = v;
  __syncthreads();
  float r = tmp[0];
  for (int w = 1; w < NT / kWave; ++w) r = fmaxf(r, tmp[w]);
  __syncthreads();
  return r;
}

template <int NT>
__device__ __forceinline__ uint32_t block_reduce_sum(uint32_t v, uint32_t* tmp) {
  v = (uint32_t)wave_sum_int((int)v);
  if (threadIdx.x % kWave == 0) tmp[threadIdx.x / kWave] = v;
  __syncthreads();
  uint32_t r = 0;
  for (int w = 0; w < NT / kWave; ++w) r += tmp[w];
  __syncthreads();
  return r;
}

template <int NT, int MAXL>
__global__ __launch_bounds__(NT) void select_kernel(const float* __restrict__ scores, int32_t tk,
                                                    int32_t top_k, int32_t* __restrict__ sel) {
  __shared__ uint32_t hist[kBins];
  __shared__ float cand[NT];
  __shared__ uint32_t red_u[NT / kWave];
  __shared__ float red_f[NT / kWave];
  __shared__ uint32_t s_bin, s_above, s_ncand;
  __shared__ float s_tau;

  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const float* srow = scores + row * tk;
  const int L = (tk + NT - 1) / NT;
  const int beg = tid * L;

  float v[MAXL];
#pragma unroll
  for (int i = 0; i < MAXL; ++i) {
    const int idx = beg + i;
    v[i] = (i < L && idx < tk) ? srow[idx] : 0.f;
  }
  auto valid = [&](int i) { return i < L && beg + i < tk; };

  // 1. value range
  float lmax = -INFINITY, lneg = -INFINITY;  // lneg = max of -v = -min
#pragma unroll
  for (int i = 0; i < MAXL; ++i)
    if (valid(i)) {
      lmax = fmaxf(lmax, v[i]);
      lneg = fmaxf(lneg, -v[i]);
    }
  const float vmax = block_reduce_max<NT>(lmax, red_f);
  const float vmin = -block_reduce_max<NT>(lneg, red_f);

  // 2. histogram over [vmin, vmax]; bin() is monotone non-decreasing in v
  for (int b = tid; b < kBins; b += NT) hist[b] = 0;
  if (tid == 0) {
    s_bin = 0;
    s_tau = vmax;
  }
  __syncthreads();
  const float inv = (vmax > vmin) ? (float)kBins / (vmax - vmin) : 0.f;
  auto bin_of = [&](float x) { return min(kBins - 1, (int)((x - vmin) * inv)); };
#pragma unroll
  for (int i = 0; i < MAXL; ++i)
    if (valid(i)) atomicAdd(&hist[bin_of(v[i])], 1u);
  __syncthreads();

  // 3. the bin in which the count from the top reaches top_k
  constexpr int BPT = kBins / NT;
  uint32_t mine = 0;
#pragma unroll
  for (int b = 0; b < BPT; ++b) mine += hist[tid * BPT + b];
  const uint32_t incl = block_inclusive_scan<NT>(mine, red_u);
  if (tid == NT - 1) s_above = incl;  // total count
  __syncthreads();
  const uint32_t all = s_above;
  __syncthreads();
  uint32_t above = all - incl;  // count in bins owned by higher threads
  for (int b = BPT - 1; b >= 0; --b) {
    const uint32_t hb = hist[tid * BPT + b];
    if (above < (uint32_t)top_k && (uint32_t)top_k <= above + hb) {
      s_bin = tid * BPT + b;
      s_above = above;
    }
    above += hb;
  }
  __syncthreads();
  const int bstar = (int)s_bin;
  const uint32_t need_in_bin = (uint32_t)top_k - s_above;  // 1 .. hist[bstar]
  const uint32_t n_in_bin = hist[bstar];

  // 4. tau = the need_in_bin-th largest value among the bin's members
  if (n_in_bin <= (uint32_t)NT) {
    if (tid == 0) s_ncand = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < MAXL; ++i)
      if (valid(i) && bin_of(v[i]) == bstar) {
        const uint32_t slot = atomicAdd(&s_ncand, 1u);
        if (slot < (uint32_t)NT) cand[slot] = v[i];
      }
    __syncthreads();
    if (tid < (int)n_in_bin) {
      const float c = cand[tid];
      uint32_t gt = 0, ge = 0;
      for (uint32_t u = 0; u < n_in_bin; ++u) {
        gt += cand[u] > c;
        ge += cand[u] >= c;
      }
      if (gt < need_in_bin && need_in_bin <= ge) s_tau = c;  // every writer stores the same value
    }
    __syncthreads();
  } else {
    // Rare: a bin holds more than NT scores (e.g. many equal values). Find tau
    // by bisection on order-preserving keys over the whole row.
    uint32_t lo_key = 0;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t trial = lo_key | (1u << bit);
      uint32_t cnt = 0;
#pragma unroll
      for (int i = 0; i < MAXL; ++i)
        if (valid(i)) cnt += float_key(v[i]) >= trial;
      if (block_reduce_sum<NT>(cnt, red_u) >= (uint32_t)top_k) lo_key = trial;
    }
    if (tid == 0) {
      const uint32_t u = (lo_key & 0x80000000u) ? (lo_key & 0x7fffffffu) : ~lo_key;
      s_tau = __uint_as_float(u);
    }
    __syncthreads();
  }
  const float tau = s_tau;

  // 5. ordered compaction: {s > tau} and the first (top_k - #{s > tau}) ties
  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int i = 0; i < MAXL; ++i)
    if (valid(i)) {
      gt += v[i] > tau;
      eq += v[i] == tau;
    }
  const uint32_t packed = (gt << 16) | eq;
  const uint32_t incl2 = block_inclusive_scan<NT>(packed, red_u);
  if (tid == NT - 1) s_above = incl2 >> 16;  // total strictly above tau
  __syncthreads();
  const uint32_t need_eq = s_above < (uint32_t)top_k ? (uint32_t)top_k - s_above : 0u;
  const uint32_t excl = incl2 - packed;
  uint32_t g = excl >> 16, e = excl & 0xffffu;
  int32_t* out = sel + row * top_k;
#pragma unroll
  for (int i = 0; i < MAXL; ++i) {
    if (!valid(i)) continue;
    if (v[i] > tau) {
      const uint32_t pos = g + min(e, need_eq);
      if (pos < (uint32_t)top_k) out[pos] = beg + i;
      ++g;
    } else if (v[i] == tau) {
      if (e < need_eq && g + e < (uint32_t)top_k) out[g + e] = beg + i;
      ++e;
    }
  }
}

}  // namespace

hipError_t launch_select(const float* qbar, const float* kbar, int32_t heads, int32_t tq,
                         int32_t tk, int32_t top_k, int32_t* sel, float* scores,
                         hipStream_t s) {
  if (heads == 0 || tq == 0) return hipSuccess;
  dim3 sgrid((tk + kScoreTile - 1) / kScoreTile, (tq + kScoreTile - 1) / kScoreTile, heads);
  hipLaunchKernelGGL(score_kernel, sgrid, dim3(256), 0, s, qbar, kbar, tq, tk, scores);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const unsigned rows = (unsigned)((int64_t)heads * tq);
  if (tk <= 256 * 4) {
    hipLaunchKernelGGL((select_kernel<256, 4>), dim3(rows), dim3(256), 0, s, scores, tk, top_k,
                       sel);
  } else if (tk <= 1024 * 8) {
    hipLaunchKernelGGL((select_kernel<1024, 8>), dim3(rows), dim3(1024), 0, s, scores, tk,
                       top_k, sel);
  } else {
    hipLaunchKernelGGL((select_kernel<1024, 32>), dim3(rows), dim3(1024), 0, s, scores, tk,
                       top_k, sel);
  }
  return hipGetLastError();
}

}  // namespace zebra
