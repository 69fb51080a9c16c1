// Selection-quality diagnostic: attention mass of every (query tile, key tile)
// block under dense softmax (gfx950).
//
// Zebra3D paper page (thelatestinai.com), Figure 2 caption, panel (b), and
// Figure 8 caption: the attention mass retained by the highest-mass 20% of
// 64x64 token blocks. For query tile i and key tile j:
//   M[h][i][j] = (1/|Q_i|) sum_{q in Q_i} sum_{k in K_j} softmax_q(scale q . k).
//
// Two passes over all keys, one workgroup per (head, query tile), one wave
// per 32 queries; scores come from bf16 MFMA 32x32x16 as transposed blocks
// S^T = K Q^T, so each lane holds one query's scores over 16 keys of a 32-key
// block (the other 16 in the lane 32 apart):
//   1. row statistics: the exact maximum m and sum l = sum 2^(c s - m) of each
//      query over all keys (c = scale log2 e), float32, running maximum;
//   2. block masses: per key tile, each query's sum of 2^(c s - m) / l over
//      the tile's keys, summed over the wave's queries by a fixed butterfly
//      and over the workgroup's waves in wave order, divided by |Q_i|.
// The K operands are read straight from global memory (a diagnostic: the
// keys of one head stay in L2). Deterministic: no atomics.
#include <algorithm>

#include "common.h"

namespace zebra {

namespace {

constexpr float kLog2eM = 1.4426950408889634f;

struct MassParams {
  const uint16_t* q;
  const uint16_t* k;
  int64_t nq, qst, qsh;
  int64_t nk, kst, ksh;
  int32_t tq, tk, q_tile, k_tile;
  float c;        // scale * log2(e)
  float2* stats;  // [H][nq] (m, l)
  float* mass;    // [H][tq][tk]
};

// Query operand of S^T = K Q^T for the wave's 32 queries: Q[q][16s + 8hh .. +7].
__device__ __forceinline__ void load_q(const MassParams& p, int h, int64_t qrow, int hh,
                                       bf16x8 (&qop)[4]) {
  const bool ok = qrow < p.nq;
  const uint16_t* qp = p.q + (int64_t)h * p.qsh + qrow * p.qst + 8 * hh;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    u32x4 w = {0u, 0u, 0u, 0u};
    if (ok) w = *(const u32x4*)(qp + 16 * s);
    qop[s] = as_bf16x8(w);
  }
}

// Scores (times c) of key block kb (32 keys) for the lane's query: register i
// holds key 32kb + 8(i/4) + 4hh + i%4; keys past nk give -inf.
__device__ __forceinline__ f32x16 score_block(const MassParams& p, int h, int64_t kb,
                                              const bf16x8 (&qop)[4], int lane) {
  const int qi = lane & 31, hh = lane >> 5;
  const int64_t krow = kb * 32 + qi;
  const bool ok = krow < p.nk;
  const uint16_t* kp = p.k + (int64_t)h * p.ksh + krow * p.kst + 8 * hh;
  f32x16 acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    u32x4 w = {0u, 0u, 0u, 0u};
    if (ok) w = *(const u32x4*)(kp + 16 * s);
    acc = mfma32(as_bf16x8(w), qop[s], acc);
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t key = kb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
    acc[i] = key < p.nk ? acc[i] * p.c : -INFINITY;
  }
  return acc;
}

__device__ __forceinline__ float partner(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                   false, false);
  // lanes 0-31 receive the partner value in the second result, lanes 32-63 in the first
  return __uint_as_float((threadIdx.x & 63) < 32 ? sw[1] : sw[0]);
}

__global__ __launch_bounds__(256) void mass_stats_kernel(MassParams p) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int h = blockIdx.y;
  const int64_t qrow = (int64_t)blockIdx.x * p.q_tile + wave * 32 + (lane & 31);
  if (wave * 32 >= p.q_tile) return;
  bf16x8 qop[4];
  load_q(p, h, qrow, lane >> 5, qop);
  float m = -INFINITY, l = 0.f;
  const int64_t nb = (p.nk + 31) / 32;
  for (int64_t kb = 0; kb < nb; ++kb) {
    const f32x16 x = score_block(p, h, kb, qop, lane);
    float bm = x[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) bm = fmaxf(bm, x[i]);
    if (bm > m) {
      l *= __builtin_amdgcn_exp2f(m - bm);  // 0 when m is -inf
      m = bm;
    }
    if (m > -INFINITY) {
#pragma unroll
      for (int i = 0; i < 16; ++i) l += __builtin_amdgcn_exp2f(x[i] - m);
    }
  }
  // combine the two lane halves (the same query, disjoint keys)
  const float m2 = partner(m), l2 = partner(l);
  const float mm = fmaxf(m, m2);
  const float ll = (m > -INFINITY ? l * __builtin_amdgcn_exp2f(m - mm) : 0.f) +
                   (m2 > -INFINITY ? l2 * __builtin_amdgcn_exp2f(m2 - mm) : 0.f);
  if (lane < 32 && qrow < p.nq) p.stats[(int64_t)h * p.nq + qrow] = float2{mm, ll};
}

__global__ __launch_bounds__(256) void mass_blocks_kernel(MassParams p) {
  __shared__ float red[2][4];
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int nw = p.q_tile / 32;
  const int h = blockIdx.y, qt = blockIdx.x;
  const int64_t qrow = (int64_t)qt * p.q_tile + wave * 32 + (lane & 31);
  const bool active = wave < nw;
  const bool qvalid = active && qrow < p.nq;
  bf16x8 qop[4];
  load_q(p, h, qrow, lane >> 5, qop);
  float m = 0.f, inv_l = 0.f;
  if (qvalid) {
    const float2 st = p.stats[(int64_t)h * p.nq + qrow];
    m = st.x;
    inv_l = 1.0f / st.y;
  }
  const int64_t q0 = (int64_t)qt * p.q_tile;
  const float inv_nq = 1.0f / (float)std::min<int64_t>(p.q_tile, p.nq - q0);
  const int bpt = p.k_tile / 32;  // 32-key blocks per key tile
  float* out = p.mass + ((int64_t)h * p.tq + qt) * p.tk;
  for (int j = 0; j < p.tk; ++j) {
    float s = 0.f;
    if (active) {
      for (int b = 0; b < bpt; ++b) {
        const f32x16 x = score_block(p, h, (int64_t)j * bpt + b, qop, lane);
#pragma unroll
        for (int i = 0; i < 16; ++i) s += __builtin_amdgcn_exp2f(x[i] - m);
      }
      s = qvalid ? (s + partner(s)) * inv_l : 0.f;  // both halves of the query
      // sum over the wave's 32 queries (lanes 0-31; 32-63 hold the same values)
#pragma unroll
      for (int o = 16; o >= 1; o >>= 1) s += __shfl_xor(s, o, kWave);
      if (lane == 0) red[j & 1][wave] = s;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      float t = 0.f;
      for (int w = 0; w < nw; ++w) t += red[j & 1][w];
      out[j] = t * inv_nq;
    }
  }
}

}  // namespace

size_t mass_workspace_bytes(int64_t n_q, int32_t heads) {
  return (size_t)heads * (size_t)n_q * sizeof(float2);
}

hipError_t launch_block_mass(const uint16_t* q, int64_t nq, int64_t qst, int64_t qsh,
                             const uint16_t* k, int64_t nk, int64_t kst, int64_t ksh,
                             int32_t heads, int32_t q_tile, int32_t k_tile, float scale,
                             float* mass, void* ws, hipStream_t s) {
  MassParams p;
  p.q = q;
  p.k = k;
  p.nq = nq;
  p.qst = qst;
  p.qsh = qsh;
  p.nk = nk;
  p.kst = kst;
  p.ksh = ksh;
  p.q_tile = q_tile;
  p.k_tile = k_tile;
  p.tq = (int32_t)((nq + q_tile - 1) / q_tile);
  p.tk = (int32_t)((nk + k_tile - 1) / k_tile);
  p.c = scale * kLog2eM;
  p.stats = (float2*)ws;
  p.mass = mass;
  if (heads == 0 || p.tq == 0) return hipSuccess;
  // 4 waves per workgroup always; waves past the query tile idle
  hipLaunchKernelGGL(mass_stats_kernel, dim3((unsigned)p.tq, heads), dim3(256), 0, s, p);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(mass_blocks_kernel, dim3((unsigned)p.tq, heads), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace zebra
