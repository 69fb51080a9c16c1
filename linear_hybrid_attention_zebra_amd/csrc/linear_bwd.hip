// Backward pass of elu+1 linear attention with the per-channel affine map (gfx950).
//
// The converted model can be refined afterwards (Zebra3D paper page, Tables
// 18-19); these are the gradients of sum(dout * out) for one linear stage,
// out = a (*) o + b, o = num / den, num = phi(q) S, den = phi(q) . z:
//   da = sum_n dout (*) o,  db = sum_n dout,  do = a (*) dout,
//   dnum = do / den,  dden = -(do . o) / den,
//   dq = (S dnum + z dden) (*) phi'(q),
//   dS = sum_n phi(q_n) dnum_n^T,  dz = sum_n phi(q_n) dden_n,
//   dv_m = dS^T phi(k_m),  dk_m = (dS v_m + dz) (*) phi'(k_m),
// with phi'(x) = 1 for x > 0 and e^x otherwise, i.e. min(phi(x), 1).
//
// The sum S dnum + z dden cancels strongly (S[c][e] / z[c] is close to o[e]
// for diffuse attention), so every product here is float32 (no bf16
// operands): the three 64x64x64 products per 64 rows run as register-tiled
// float32 GEMMs from LDS, 4x4 outputs per thread. Kernels:
//  1. (forward state S, z: the forward's state and reduce kernels)
//  2. query pass: per (head, row range) workgroup, for each 64-row block:
//     num = phi S, den, o, dnum, dden, dq = (dnum S^T + z dden) (*) phi';
//     accumulates dS, dz, da, db of its rows in registers, written once;
//  3. reduce of the workgroup partials in a fixed order (float64);
//  4. key pass: dv = phi(k) dS, dk = (v dS^T + dz) (*) phi'(k).
// No atomics: bitwise reproducible.
#include <algorithm>

#include "common.h"

namespace zebra {

namespace {

constexpr int kLd = 68;  // LDS row stride in floats (64 + 4 keeps float4 alignment)
constexpr int kPartFloats = kHeadDim * kHeadDim + 3 * kHeadDim;  // dS, dz, da, db
constexpr int kRowsPerBlock = 64;

__device__ __forceinline__ float phi_f(float x) { return x > 0.f ? x + 1.f : __expf(x); }

// 8 channels of a row of a bf16 or float32 tensor (16-byte aligned pieces)
__device__ __forceinline__ void load8(const void* base, int64_t elem, bool f32, float* out) {
  if (f32) {
    const f32x4 a = *(const f32x4*)((const float*)base + elem);
    const f32x4 b = *(const f32x4*)((const float*)base + elem + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[i] = a[i];
      out[4 + i] = b[i];
    }
  } else {
    const u32x4 w = *(const u32x4*)((const uint16_t*)base + elem);
    const uint32_t e[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = bf16lo(e[i]);
      out[2 * i + 1] = bf16hi(e[i]);
    }
  }
}

// 4 consecutive channels of a row
__device__ __forceinline__ void store4(void* base, int64_t elem, bool f32, const float* v) {
  if (f32) {
    *(f32x4*)((float*)base + elem) = f32x4{v[0], v[1], v[2], v[3]};
  } else {
    *(u32x2*)((uint16_t*)base + elem) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  }
}

// acc[i][j] += sum_k A[k][r0 + i] B[k][c0 + j]; A, B in LDS with row stride kLd
__device__ __forceinline__ void gemm4x4(const float* A, const float* B, int r0, int c0,
                                        float (&acc)[4][4]) {
#pragma unroll 8
  for (int kk = 0; kk < kHeadDim; ++kk) {
    const f32x4 a = *(const f32x4*)(A + kk * kLd + r0);
    const f32x4 b = *(const f32x4*)(B + kk * kLd + c0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
  }
}

struct BwdQParams {
  const uint16_t* q;
  int64_t nq, qst, qsh;
  const void* dout;
  int64_t dst, dsh;
  void* dq;
  int64_t gst, gsh;
  int32_t g_f32;
  const float* state;  // [H][S | z]
  const float* aff_a;  // [H][64] or null
  int64_t rows_per_wg;
  float* part;  // [H][n_wg][kPartFloats]
};

__global__ __launch_bounds__(256) void linear_bwd_query_kernel(BwdQParams p) {
  __shared__ float S[kHeadDim * kLd];    // S[c][e]
  __shared__ float St[kHeadDim * kLd];   // S^T[e][c]
  __shared__ float phT[kHeadDim * kLd];  // phi^T[c][r]
  __shared__ float ph[kRowsPerBlock * kLd];   // phi[r][c]
  __shared__ float dnT[kHeadDim * kLd];  // dnum^T[e][r]
  __shared__ float dn[kRowsPerBlock * kLd];   // dnum[r][e]
  __shared__ float zs[kHeadDim], as[kHeadDim], den_s[kRowsPerBlock], dden_s[kRowsPerBlock];
  __shared__ float red[16][2 * kHeadDim];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int h = blockIdx.y, wg = blockIdx.x;
  const float* st = p.state + (int64_t)h * (kHeadDim * kHeadDim + kHeadDim);
  for (int e = tid; e < kHeadDim * kHeadDim; e += 256) {
    const int c = e / kHeadDim, j = e % kHeadDim;
    S[c * kLd + j] = st[e];
    St[j * kLd + c] = st[e];
  }
  if (tid < kHeadDim) {
    zs[tid] = st[kHeadDim * kHeadDim + tid];
    as[tid] = p.aff_a != nullptr ? p.aff_a[h * kHeadDim + tid] : 1.f;
  }
  float dS[4][4] = {}, da[4] = {}, db[4] = {}, dz[4] = {};
  const int64_t row0 = (int64_t)wg * p.rows_per_wg;
  const int64_t row1 = std::min<int64_t>(p.nq, row0 + p.rows_per_wg);
  const uint16_t* qh = p.q + (int64_t)h * p.qsh;
  const bool gf = p.g_f32 != 0;
  const int r0 = 4 * ty, c0 = 4 * tx;  // this thread's 4x4 outputs
  for (int64_t rb = row0; rb < row1; rb += kRowsPerBlock) {
    __syncthreads();  // the previous block's tiles are consumed; state is loaded
    // phi(q) tiles in both layouts; rows past the end are zero
    for (int e = tid; e < kRowsPerBlock * 8; e += 256) {
      const int r = e >> 3, c8 = (e & 7) * 8;
      float f[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (rb + r < row1) {
        load8(qh, (rb + r) * p.qst + c8, false, f);
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = phi_f(f[i]);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        ph[r * kLd + c8 + i] = f[i];
        phT[(c8 + i) * kLd + r] = f[i];
      }
    }
    __syncthreads();
    if (tid < kRowsPerBlock) {  // den = phi . z per row
      float d = 0.f;
      for (int c = 0; c < kHeadDim; ++c) d = __builtin_fmaf(ph[tid * kLd + c], zs[c], d);
      den_s[tid] = d;
    }
    // num = phi S: rows r0.., channels c0..
    float num[4][4] = {};
    gemm4x4(phT, S, r0, c0, num);
    __syncthreads();
    // o, do, dnum per row; dot(do, o) across the 16 threads of a row group
    float dnum[4][4], dot[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t row = rb + r0 + i;
      const bool ok = row < row1;
      float g[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (ok) {  // 4 channels: load the 8-channel piece and take the half
        load8(p.dout, (int64_t)h * p.dsh + row * p.dst + (c0 & ~7), gf, g);
      }
      const float* gd = g + (c0 & 4);
      const float inv = ok ? 1.f / den_s[r0 + i] : 0.f;
      dot[i] = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float o = num[i][j] * inv;
        const float dov = as[c0 + j] * gd[j];
        da[j] = __builtin_fmaf(gd[j], o, da[j]);
        db[j] += gd[j];
        dot[i] = __builtin_fmaf(dov, o, dot[i]);
        dnum[i][j] = dov * inv;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int m = 1; m < 16; m <<= 1) dot[i] += __shfl_xor(dot[i], m, 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (tx == 0) {
        const int64_t row = rb + r0 + i;
        dden_s[r0 + i] = row < row1 ? -dot[i] / den_s[r0 + i] : 0.f;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        dn[(r0 + i) * kLd + c0 + j] = dnum[i][j];
        dnT[(c0 + j) * kLd + r0 + i] = dnum[i][j];
      }
    }
    __syncthreads();
    // dq = (dnum S^T + z dden) (*) phi': rows r0.., channels c0..
    float dphi[4][4] = {};
    gemm4x4(dnT, St, r0, c0, dphi);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t row = rb + r0 + i;
      if (row >= row1) continue;
      float g[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float f = ph[(r0 + i) * kLd + c0 + j];
        g[j] = (dphi[i][j] + zs[c0 + j] * dden_s[r0 + i]) * fminf(f, 1.f);
      }
      store4(p.dq, (int64_t)h * p.gsh + row * p.gst + c0, gf, g);
    }
    // dS += phi^T dnum: state rows (channels of phi) r0.., columns c0..
    gemm4x4(ph, dn, r0, c0, dS);
    // dz += phi^T dden for channels c0.. (threads of row group 0)
    if (ty == 0)
      for (int r = 0; r < kRowsPerBlock; ++r)
#pragma unroll
        for (int j = 0; j < 4; ++j) dz[j] = __builtin_fmaf(ph[r * kLd + c0 + j], dden_s[r], dz[j]);
  }
  // partials: dS by thread tiles; da, db summed over the 16 row groups in order
  float* out = p.part + ((int64_t)h * gridDim.x + wg) * kPartFloats;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) out[(r0 + i) * kHeadDim + c0 + j] = dS[i][j];
  if (ty == 0)
#pragma unroll
    for (int j = 0; j < 4; ++j) out[kHeadDim * kHeadDim + c0 + j] = dz[j];
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    red[ty][c0 + j] = da[j];
    red[ty][kHeadDim + c0 + j] = db[j];
  }
  __syncthreads();
  if (tid < 2 * kHeadDim) {
    float s = 0.f;
    for (int g = 0; g < 16; ++g) s += red[g][tid];
    out[kHeadDim * kHeadDim + kHeadDim + tid] = s;
  }
}

// Sums the workgroup partials in order (float64): dS and dz into the state
// workspace, da and db into the caller's outputs.
__global__ __launch_bounds__(256) void linear_bwd_reduce_kernel(const float* __restrict__ part,
                                                                int32_t n_wg,
                                                                float* __restrict__ dstate,
                                                                float* __restrict__ d_scale,
                                                                float* __restrict__ d_bias) {
  const int h = blockIdx.y;
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= kPartFloats) return;
  const float* ph = part + (int64_t)h * n_wg * kPartFloats + e;
  double s = 0.0;
  for (int w = 0; w < n_wg; ++w) s += (double)ph[(int64_t)w * kPartFloats];
  const int sd = kHeadDim * kHeadDim + kHeadDim;
  if (e < sd) {
    dstate[(int64_t)h * sd + e] = (float)s;
  } else if (e < sd + kHeadDim) {
    if (d_scale != nullptr) d_scale[h * kHeadDim + e - sd] = (float)s;
  } else if (d_bias != nullptr) {
    d_bias[h * kHeadDim + e - sd - kHeadDim] = (float)s;
  }
}

struct BwdKParams {
  const uint16_t* k;
  const uint16_t* v;
  int64_t nk, kst, ksh;
  void* dk;
  void* dv;
  int64_t gst, gsh;
  int32_t g_f32;
  const float* dstate;  // [H][dS | dz]
};

__global__ __launch_bounds__(256) void linear_bwd_key_kernel(BwdKParams p) {
  __shared__ float dS[kHeadDim * kLd];   // dS[c][e]
  __shared__ float dSt[kHeadDim * kLd];  // dS^T[e][c]
  __shared__ float phT[kHeadDim * kLd];  // phi(k)^T[c][m]
  __shared__ float ph[kRowsPerBlock * kLd];  // phi(k)[m][c]
  __shared__ float vT[kHeadDim * kLd];   // v^T[e][m]
  __shared__ float dzs[kHeadDim];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int h = blockIdx.y;
  const float* st = p.dstate + (int64_t)h * (kHeadDim * kHeadDim + kHeadDim);
  for (int e = tid; e < kHeadDim * kHeadDim; e += 256) {
    const int c = e / kHeadDim, j = e % kHeadDim;
    dS[c * kLd + j] = st[e];
    dSt[j * kLd + c] = st[e];
  }
  if (tid < kHeadDim) dzs[tid] = st[kHeadDim * kHeadDim + tid];
  const uint16_t* kh = p.k + (int64_t)h * p.ksh;
  const uint16_t* vh = p.v + (int64_t)h * p.ksh;
  const bool gf = p.g_f32 != 0;
  const int r0 = 4 * ty, c0 = 4 * tx;
  for (int64_t mb = (int64_t)blockIdx.x * kRowsPerBlock; mb < p.nk;
       mb += (int64_t)gridDim.x * kRowsPerBlock) {
    __syncthreads();
    for (int e = tid; e < kRowsPerBlock * 8; e += 256) {
      const int m = e >> 3, c8 = (e & 7) * 8;
      float f[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      float w[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (mb + m < p.nk) {
        load8(kh, (mb + m) * p.kst + c8, false, f);
        load8(vh, (mb + m) * p.kst + c8, false, w);
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = phi_f(f[i]);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        ph[m * kLd + c8 + i] = f[i];
        phT[(c8 + i) * kLd + m] = f[i];
        vT[(c8 + i) * kLd + m] = w[i];
      }
    }
    __syncthreads();
    float dv[4][4] = {}, dkp[4][4] = {};
    gemm4x4(phT, dS, r0, c0, dv);   // dv[m][e] = sum_c phi[m][c] dS[c][e]
    gemm4x4(vT, dSt, r0, c0, dkp);  // (v dS^T)[m][c] = sum_e v[m][e] dS[c][e]
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t m = mb + r0 + i;
      if (m >= p.nk) continue;
      float g[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        g[j] = (dkp[i][j] + dzs[c0 + j]) * fminf(ph[(r0 + i) * kLd + c0 + j], 1.f);
      store4(p.dk, (int64_t)h * p.gsh + m * p.gst + c0, gf, g);
      store4(p.dv, (int64_t)h * p.gsh + m * p.gst + c0, gf, dv[i]);
    }
  }
}

void bwd_chunking(int64_t nq, int32_t heads, int32_t& n_wg, int64_t& rows) {
  // about 2,048 workgroups in all, each over whole 64-row blocks
  const int64_t per_head = std::max<int64_t>(1, 2048 / std::max(1, heads));
  rows = std::max<int64_t>(kRowsPerBlock,
                           ((nq + per_head - 1) / per_head + kRowsPerBlock - 1) /
                               kRowsPerBlock * kRowsPerBlock);
  n_wg = (int32_t)std::max<int64_t>(1, (nq + rows - 1) / rows);
}

}  // namespace

size_t linear_bwd_workspace_bytes(int64_t n_q, int64_t n_kv, int32_t heads) {
  int32_t n_wg;
  int64_t rows;
  bwd_chunking(n_q, heads, n_wg, rows);
  const size_t fwd = linear_workspace_bytes(n_kv, heads);  // partial states + S, z
  const size_t part = (size_t)heads * n_wg * kPartFloats * sizeof(float);
  const size_t dstate = (size_t)heads * (kHeadDim * kHeadDim + kHeadDim) * sizeof(float);
  return fwd + part + dstate;
}

hipError_t launch_linear_bwd(const uint16_t* q, int64_t nq, int64_t qst, int64_t qsh,
                             const uint16_t* k, const uint16_t* v, int64_t nk, int64_t kst,
                             int64_t ksh, int32_t heads, const float* aff_scale,
                             const void* dout, int64_t dst, int64_t dsh, void* dq, int64_t qgst,
                             int64_t qgsh, void* dk, void* dv, int64_t kgst, int64_t kgsh,
                             bool g_f32, float* d_scale, float* d_bias, void* ws,
                             hipStream_t s) {
  if (heads == 0) return hipSuccess;
  float* state = nullptr;
  hipError_t err = launch_linear_state(k, v, nk, kst, ksh, heads, ws, &state, s);
  if (err != hipSuccess) return err;
  int32_t n_wg;
  int64_t rows;
  bwd_chunking(nq, heads, n_wg, rows);
  uint8_t* w = (uint8_t*)ws + linear_workspace_bytes(nk, heads);
  float* part = (float*)w;
  float* dstate = part + (size_t)heads * n_wg * kPartFloats;
  BwdQParams pq{q, nq, qst, qsh, dout, dst, dsh, dq, qgst, qgsh, g_f32 ? 1 : 0,
                state, aff_scale, rows, part};
  hipLaunchKernelGGL(linear_bwd_query_kernel, dim3(n_wg, heads), dim3(256), 0, s, pq);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(linear_bwd_reduce_kernel, dim3((kPartFloats + 255) / 256, heads), dim3(256),
                     0, s, part, n_wg, dstate, d_scale, d_bias);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (nk == 0) return hipSuccess;
  BwdKParams pk{k, v, nk, kst, ksh, dk, dv, kgst, kgsh, g_f32 ? 1 : 0, dstate};
  const int64_t blocks = std::min<int64_t>((nk + kRowsPerBlock - 1) / kRowsPerBlock,
                                           std::max<int64_t>(1, 2048 / heads));
  hipLaunchKernelGGL(linear_bwd_key_kernel, dim3((unsigned)blocks, heads), dim3(256), 0, s, pk);
  return hipGetLastError();
}

}  // namespace zebra
