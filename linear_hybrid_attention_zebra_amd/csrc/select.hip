// Tile selection: pooled-query . pooled-key scores, then top-k per query tile.
//
// The tile-sparse stage computes only selected blocks (news.hamidun.com
// article "Zebra3D speeds up 3D reconstruction...", section "How Zebra3D
// works"). Score of query tile i and key tile j: s_ij = qbar_i . kbar_j in
// float32. Each (head, i) keeps the top_k key tiles under the order
// (s_ij descending, j ascending) and emits them in ascending order.
//
// Two kernels:
//  1. score_kernel: a K=64 float32 GEMM on float32 MFMAs, 128x128 output
//     tile per workgroup, operands staged in LDS; every element has the same
//     fixed summation order. Score rows are padded to 32 floats.
//  2. select_kernel: one wave per (head, query tile), no workgroup barriers.
//     The k-th largest value tau is found exactly: min/max, a 2048-bin
//     histogram on the value range (a monotone binning, so equal scores share
//     a bin), the bin where the count from the top crosses k, then an exact
//     rank among that bin's members (bisection on order-preserving keys when
//     the bin is crowded). Kept tiles are {s > tau} plus the lowest-indexed
//     ties at tau, written in index order through wave prefix sums. No sort,
//     no float atomics; the result does not depend on scheduling.
#include "common.h"

namespace zebra {

namespace {

constexpr int kScoreTile = 128;  // output tile edge of score_kernel

// One 128x128 tile of s = qbar kbar^T per workgroup, a 64x64 quarter per
// wave, on float32 MFMAs (32x32x2: exact float32 products, float32 sums).
// Both operand tiles sit row-major in LDS (rows padded to 68 floats, so the
// 16-byte reads of 16 consecutive rows hit distinct banks). MFMA step t
// contracts channels t (lane half 0) and 32 + t (lane half 1), t = 0..31 in
// order: every output element has the same fixed summation order, and
// integer-valued inputs give exact scores. Score rows are ld floats apart, ld
// a multiple of 32, so each 32-lane store fills one 128-byte line.
__global__ __launch_bounds__(256) void score_kernel(const float* __restrict__ qbar,
                                                    const float* __restrict__ kbar, int32_t tq,
                                                    int32_t tk, int32_t ld,
                                                    float* __restrict__ scores) {
  constexpr int T = kScoreTile, LD = kHeadDim + 4;
  __shared__ __attribute__((aligned(16))) float qs[T * LD];
  __shared__ __attribute__((aligned(16))) float ks[T * LD];
  const int h = blockIdx.z;
  const int i0 = blockIdx.y * T;
  const int j0 = blockIdx.x * T;
  const int tid = threadIdx.x;
  const float* qh = qbar + (int64_t)h * tq * kHeadDim;
  const float* kh = kbar + (int64_t)h * tk * kHeadDim;
  // 128 rows x 16 float4 per operand: 8 float4 of each per thread
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int e = tid + 256 * u;
    const int r = e >> 4, c4 = e & 15;
    f32x4 qv = {0.f, 0.f, 0.f, 0.f}, kv = {0.f, 0.f, 0.f, 0.f};
    if (i0 + r < tq) qv = *(const f32x4*)(qh + (int64_t)(i0 + r) * kHeadDim + 4 * c4);
    if (j0 + r < tk) kv = *(const f32x4*)(kh + (int64_t)(j0 + r) * kHeadDim + 4 * c4);
    *(f32x4*)&qs[r * LD + 4 * c4] = qv;
    *(f32x4*)&ks[r * LD + 4 * c4] = kv;
  }
  __syncthreads();
  const int wave = tid / kWave, lane = tid % kWave;
  const int hh = lane >> 5, l32 = lane & 31;
  const int wr = 64 * (wave >> 1), wc = 64 * (wave & 1);  // the wave's quarter
  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.f;
#pragma unroll
  for (int u = 0; u < 8; ++u) {  // channels 32 hh + 4 u .. +3: steps t = 4u .. 4u+3
    f32x4 qa[2], kb[2];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      qa[a] = *(const f32x4*)&qs[(wr + 32 * a + l32) * LD + 32 * hh + 4 * u];
      kb[a] = *(const f32x4*)&ks[(wc + 32 * a + l32) * LD + 32 * hh + 4 * u];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x2f32(qa[a][e], kb[b][e], acc[a][b], 0, 0, 0);
  }
  // lane l holds column l % 32 and rows 8 (v / 4) + 4 (l / 32) + v % 4 of a block
  float* out = scores + (int64_t)h * tq * ld;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int j = j0 + wc + 32 * b + l32;
      if (j >= tk) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int i = i0 + wr + 32 * a + 8 * (v >> 2) + 4 * hh + (v & 3);
        if (i < tq) out[(int64_t)i * ld + j] = acc[a][b][v];
      }
    }
}

constexpr int kBins = 2048;
constexpr int kRowsPerGroup = 4;  // one wave per row
constexpr int kMaxCand = 256;     // members of the threshold bin ranked exactly

__device__ __forceinline__ float wave_min(float v) {
  for (int o = 32; o >= 1; o >>= 1) v = fminf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Inclusive prefix sum over the wave's 64 lanes.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, int lane) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const uint32_t u = __shfl_up(v, o, kWave);
    if (lane >= o) v += u;
  }
  return v;
}

// Row elements in chunks of 256: lane l holds elements 256c + 4l .. +3 (index
// order = chunk, lane, element), 16-byte loads when the row allows them.
struct RowReader {
  const float* row;
  int32_t n;
  bool vec;
  __device__ __forceinline__ void load(int c, int lane, float (&x)[4]) const {
    const int i0 = 256 * c + 4 * lane;
    if (vec && i0 + 3 < n) {
      const f32x4 w = *(const f32x4*)(row + i0);
      x[0] = w.x;
      x[1] = w.y;
      x[2] = w.z;
      x[3] = w.w;
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) x[u] = i0 + u < n ? row[i0 + u] : 0.f;
    }
  }
};

// Visits chunks 0 .. n-1 in order; the loads of kB chunks go out together
// (a pass over a row is otherwise one load latency per chunk).
template <class F>
__device__ __forceinline__ void for_chunks(const RowReader& rd, int nchunks, int lane, F&& f) {
  constexpr int kB = 4;
  int c = 0;
  for (; c + kB <= nchunks; c += kB) {
    float x[kB][4];
#pragma unroll
    for (int j = 0; j < kB; ++j) rd.load(c + j, lane, x[j]);
#pragma unroll
    for (int j = 0; j < kB; ++j) f(c + j, x[j]);
  }
  for (; c < nchunks; ++c) {
    float x[4];
    rd.load(c, lane, x);
    f(c, x);
  }
}

// One wave per (head, query tile) row; no workgroup barriers. Passes over the
// row (re-read from L2): value range; a 2048-bin monotone histogram in LDS;
// the bin where the count from the top reaches top_k; the exact threshold tau
// among that bin's members (or by bisection on order-preserving keys when the
// bin holds more than kMaxCand values, e.g. many equal scores); then an
// ordered compaction of {s > tau} plus the lowest-indexed ties at tau.
__global__ __launch_bounds__(kRowsPerGroup * kWave) void select_kernel(
    const float* __restrict__ scores, int64_t n_rows, int32_t tk, int32_t ld, int32_t top_k,
    int32_t* __restrict__ sel) {
  __shared__ uint32_t hist_all[kRowsPerGroup][kBins];
  __shared__ float cand_all[kRowsPerGroup][kMaxCand];
  __shared__ uint32_t ncand_all[kRowsPerGroup];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerGroup + wave;
  if (row >= n_rows) return;  // whole wave; no barriers follow
  uint32_t* hist = hist_all[wave];
  float* cand = cand_all[wave];
  const RowReader rd{scores + row * ld, tk, true};  // rows start 128-byte aligned
  const int nchunks = (tk + 255) / 256;
  auto valid = [&](int c, int u) { return 256 * c + 4 * lane + u < tk; };

  // 1. value range
  float lmax = -INFINITY, lmin = INFINITY;
  for_chunks(rd, nchunks, lane, [&](int c, const float (&x)[4]) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (valid(c, u)) {
        lmax = fmaxf(lmax, x[u]);
        lmin = fminf(lmin, x[u]);
      }
  });
  const float vmax = wave_max(lmax), vmin = wave_min(lmin);

  // 2. histogram; bin() is monotone non-decreasing in the value
  for (int b = lane; b < kBins; b += kWave) hist[b] = 0u;
  const float inv = (vmax > vmin) ? (float)kBins / (vmax - vmin) : 0.f;
  auto bin_of = [&](float x) { return min(kBins - 1, (int)((x - vmin) * inv)); };
  for_chunks(rd, nchunks, lane, [&](int c, const float (&x)[4]) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (valid(c, u)) atomicAdd(&hist[bin_of(x[u])], 1u);
  });

  // 3. the bin where the count from the top reaches top_k: lane l owns bins
  // 32(63-l) .. 32(63-l)+31, so lane order is descending value order
  constexpr int BPL = kBins / kWave;
  const int b0 = BPL * (kWave - 1 - lane);
  uint32_t mine = 0;
#pragma unroll 8
  for (int b = 0; b < BPL; ++b) mine += hist[b0 + b];
  const uint32_t incl = wave_incl_scan(mine, lane);  // count in bins >= b0
  uint32_t above = incl - mine;                      // count in bins above this lane's
  int bstar = -1;
  uint32_t above_star = 0;
  if (above < (uint32_t)top_k && (uint32_t)top_k <= incl) {
    for (int b = BPL - 1; b >= 0; --b) {
      const uint32_t hb = hist[b0 + b];
      if (above < (uint32_t)top_k && (uint32_t)top_k <= above + hb) {
        bstar = b0 + b;
        above_star = above;
        break;
      }
      above += hb;
    }
  }
  // exactly one lane found it; broadcast
  const uint64_t who = __ballot(bstar >= 0);
  const int src = __ffsll((unsigned long long)who) - 1;
  bstar = __shfl(bstar, src, kWave);
  above_star = __shfl(above_star, src, kWave);
  const uint32_t need_in_bin = (uint32_t)top_k - above_star;  // 1 .. hist[bstar]
  const uint32_t n_in_bin = hist[bstar];

  // 4. tau = the need_in_bin-th largest value of the bin
  float tau;
  if (n_in_bin <= (uint32_t)kMaxCand) {
    if (lane == 0) ncand_all[wave] = 0u;
    for_chunks(rd, nchunks, lane, [&](int c, const float (&x)[4]) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (valid(c, u) && bin_of(x[u]) == bstar) {
          const uint32_t slot = atomicAdd(&ncand_all[wave], 1u);
          cand[slot] = x[u];
        }
    });
    float t = -INFINITY;
    bool found = false;
    for (uint32_t i = lane; i < n_in_bin; i += kWave) {
      const float ci = cand[i];
      uint32_t gt = 0, ge = 0;
      for (uint32_t j = 0; j < n_in_bin; ++j) {
        gt += cand[j] > ci;
        ge += cand[j] >= ci;
      }
      if (gt < need_in_bin && need_in_bin <= ge) {
        t = ci;  // every lane that finds it holds the same value
        found = true;
      }
    }
    const uint64_t w2 = __ballot(found);
    tau = __shfl(t, __ffsll((unsigned long long)w2) - 1, kWave);
  } else {
    // many equal or nearly equal scores: bisection on order-preserving keys
    uint32_t lo_key = 0;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t trial = lo_key | (1u << bit);
      uint32_t cnt = 0;
      for (int c = 0; c < nchunks; ++c) {
        float x[4];
        rd.load(c, lane, x);
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (valid(c, u)) cnt += float_key(x[u]) >= trial;
      }
      if ((uint32_t)wave_sum_int((int)cnt) >= (uint32_t)top_k) lo_key = trial;
    }
    const uint32_t u = (lo_key & 0x80000000u) ? (lo_key & 0x7fffffffu) : ~lo_key;
    tau = __uint_as_float(u);
  }

  // 5. ordered compaction: {s > tau}, then ties at tau in index order while
  // fewer than top_k are kept. Every score in a bin above bstar exceeds tau
  // (the binning is monotone), so n_gt needs a pass only after bisection.
  uint32_t n_gt = 0;
  if (n_in_bin <= (uint32_t)kMaxCand) {
    uint32_t m = 0;
    for (uint32_t i = lane; i < n_in_bin; i += kWave) m += cand[i] > tau;
    n_gt = above_star + (uint32_t)wave_sum_int((int)m);
  } else {
    for (int c = 0; c < nchunks; ++c) {
      float x[4];
      rd.load(c, lane, x);
#pragma unroll
      for (int u = 0; u < 4; ++u) n_gt += valid(c, u) && x[u] > tau;
    }
    n_gt = (uint32_t)wave_sum_int((int)n_gt);
  }
  const uint32_t need_eq = n_gt < (uint32_t)top_k ? (uint32_t)top_k - n_gt : 0u;
  int32_t* out = sel + row * top_k;
  uint32_t base = 0, ties = 0;  // kept so far, ties seen so far (uniform)
  for_chunks(rd, nchunks, lane, [&](int c, const float (&x)[4]) {
    uint32_t g = 0, e = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (valid(c, u)) {
        g += x[u] > tau;
        e += x[u] == tau;
      }
    const uint32_t packed = (g << 16) | e;
    const uint32_t inc = wave_incl_scan(packed, lane);
    const uint32_t exc = inc - packed;
    uint32_t eg = exc >> 16, ee = exc & 0xffffu;  // before this lane, in this chunk
    const uint32_t tot = __shfl(inc, kWave - 1, kWave);
    // kept before this lane's first element: strictly-greater ones plus the
    // ties still within the budget
    const uint32_t ties_before = ties + ee;
    uint32_t pos = base + eg + min(ties_before, need_eq) - min(ties, need_eq);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (!valid(c, u)) continue;
      const int32_t idx = 256 * c + 4 * lane + u;
      if (x[u] > tau) {
        if (pos < (uint32_t)top_k) out[pos] = idx;
        ++pos;
      } else if (x[u] == tau) {
        if (ties + ee < need_eq) {
          if (pos < (uint32_t)top_k) out[pos] = idx;
          ++pos;
        }
        ++ee;
      }
    }
    const uint32_t tg = tot >> 16, te = tot & 0xffffu;
    base += tg + min(ties + te, need_eq) - min(ties, need_eq);
    ties += te;
  });
}

}  // namespace

hipError_t launch_select(const float* qbar, const float* kbar, int32_t heads, int32_t tq,
                         int32_t tk, int32_t top_k, int32_t* sel, float* scores,
                         hipStream_t s) {
  if (heads == 0 || tq == 0) return hipSuccess;
  dim3 sgrid((tk + kScoreTile - 1) / kScoreTile, (tq + kScoreTile - 1) / kScoreTile, heads);
  const int32_t ld = score_row_stride(tk);
  hipLaunchKernelGGL(score_kernel, sgrid, dim3(256), 0, s, qbar, kbar, tq, tk, ld, scores);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t rows = (int64_t)heads * tq;
  hipLaunchKernelGGL(select_kernel, dim3((unsigned)((rows + kRowsPerGroup - 1) / kRowsPerGroup)),
                     dim3(kRowsPerGroup * kWave), 0, s, scores, rows, tk, ld, top_k, sel);
  return hipGetLastError();
}

}  // namespace zebra
