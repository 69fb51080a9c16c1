// elu+1 linear attention with the per-channel affine map (gfx950).
//
// Tolerant stages run linear(-centered) attention followed by a closed-form
// affine map (Zebra3D paper page, thelatestinai.com: Abstract; Table 3(a)).
// With phi(x) = elu(x) + 1:
//   S = sum_n phi(k_n) v_n^T,  z = sum_n phi(k_n),
//   out_m = a (*) (phi(q_m)^T S) / (phi(q_m)^T z) + b.
//
// Three kernels, all streaming at HBM rate:
//  1. state: per (head, token chunk) partial S and z. K and V blocks of 64
//     tokens go to LDS row-major; phi(K) is formed in float32 and split into
//     bf16 hi + lo parts (phi = hi + lo to ~2^-17), so two bf16 MFMAs give a
//     float32-grade product. The contraction runs over tokens, so both MFMA
//     operands are read token-transposed with ds_read_b64_tr_b16. Each of the
//     4 waves owns one 32x32 quarter of S.
//  2. reduce: partial states summed over chunks in a fixed order (float64),
//     then the affine map folded into the state: a (*) (phi^T S)/(phi^T z) + b
//     = phi^T (S diag(a) + z b^T) / (phi^T z). The folded state is stored as
//     bf16 hi/lo MFMA A-operands.
//  3. apply: O^T = S'^T phi(Q)^T with three bf16 MFMAs per product (hi.hi,
//     hi.lo, lo.hi); the denominator phi(q).z is a float32 dot product.
// No atomics: the result is bitwise reproducible.
#include <algorithm>

#include "common.h"

namespace zebra {

namespace {

typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr int kBlockTok = 64;
constexpr int kStateFloats = kHeadDim * kHeadDim + kHeadDim;  // S then z
constexpr int kTargetStateBlocks = 2048;

// Byte offset of 16-byte chunk `chunk` of 128-byte row `row`: chunks are
// XORed with a function of the row that keeps the transposed operand reads
// (4 consecutive rows, 64 contiguous bytes each) bank-conflict free.
__device__ __forceinline__ uint32_t swz(int row, int chunk) {
  const int f = (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
  return (uint32_t)(row * 128 + ((chunk ^ f) << 4));
}

__device__ __forceinline__ float phi(float x) { return x > 0.f ? x + 1.f : __expf(x); }

// phi values f[0..7] -> bf16 hi = bf16(f) and lo = bf16(f - hi), 8 per vector
__device__ __forceinline__ void split8(const float* f, u32x4& hi, u32x4& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
    l[i] = pack_bf16x2(f[2 * i] - bf16lo(h[i]), f[2 * i + 1] - bf16hi(h[i]));
  }
  hi = u32x4{h[0], h[1], h[2], h[3]};
  lo = u32x4{l[0], l[1], l[2], l[3]};
}

__device__ __forceinline__ u32x2 tr_read(const uint8_t* lds, uint32_t off) {
  const i16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(lds + off));
  return __builtin_bit_cast(u32x2, t);
}

// Offset of the 8-byte piece that lane `lane` contributes to a transposed read
// returning tokens kbase..kbase+3 of channels 32*cb + lane%32.
__device__ __forceinline__ uint32_t tr_offset(int lane, int kbase, int cb) {
  const int G = lane >> 4, S = lane & 15;
  const int col = 32 * cb + 16 * (G & 1) + 4 * (S & 3);
  return swz(kbase + (S >> 2), col >> 3) + ((col & 7) ? 8 : 0);
}

__global__ __launch_bounds__(256) void linear_state_kernel(const uint16_t* __restrict__ k,
                                                           const uint16_t* __restrict__ v,
                                                           int64_t nk, int64_t kst, int64_t ksh,
                                                           int64_t chunk_tok, int32_t nchunks,
                                                           float* __restrict__ partial) {
  __shared__ __attribute__((aligned(16))) uint8_t khi[kBlockTok * 128];
  __shared__ __attribute__((aligned(16))) uint8_t klo[kBlockTok * 128];
  __shared__ __attribute__((aligned(16))) uint8_t vls[kBlockTok * 128];
  __shared__ float zred[256][9];

  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int chunk = blockIdx.x, h = blockIdx.y;
  const int64_t t0 = (int64_t)chunk * chunk_tok;
  const int64_t t1 = std::min(nk, t0 + chunk_tok);
  const uint16_t* kh = k + (int64_t)h * ksh;
  const uint16_t* vh = v + (int64_t)h * ksh;
  const int cb = wave >> 1, eb = wave & 1;  // this wave's 32x32 quarter of S

  f32x16 acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  float z8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};

  for (int64_t b0 = t0; b0 < t1; b0 += kBlockTok) {
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int e = tid + 256 * u;
      const int r = e >> 3, c = e & 7;
      const int64_t tok = b0 + r;
      u32x4 kw = {0u, 0u, 0u, 0u}, vw = {0u, 0u, 0u, 0u};
      const bool ok = tok < t1;
      if (ok) {
        kw = *(const u32x4*)(kh + tok * kst + 8 * c);
        vw = *(const u32x4*)(vh + tok * kst + 8 * c);
      }
      float f[8];
      f[0] = phi(bf16lo(kw.x));
      f[1] = phi(bf16hi(kw.x));
      f[2] = phi(bf16lo(kw.y));
      f[3] = phi(bf16hi(kw.y));
      f[4] = phi(bf16lo(kw.z));
      f[5] = phi(bf16hi(kw.z));
      f[6] = phi(bf16lo(kw.w));
      f[7] = phi(bf16hi(kw.w));
      if (!ok) {
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = 0.f;  // padded tokens add nothing
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) z8[i] += f[i];
      u32x4 hi, lo;
      split8(f, hi, lo);
      *(u32x4*)(khi + swz(r, c)) = hi;
      *(u32x4*)(klo + swz(r, c)) = lo;
      *(u32x4*)(vls + swz(r, c)) = vw;
    }
    __syncthreads();
    // S[c][e] += sum_n phi(K)[n][c] V[n][e]: A = phi(K)^T (channels x tokens),
    // B = V (tokens x channels); element j of a lane half = token 8*half + j.
#pragma unroll
    for (int s = 0; s < kBlockTok / 16; ++s) {
      const int kb0 = 16 * s + 8 * (lane >> 5);
      const u32x2 ah0 = tr_read(khi, tr_offset(lane, kb0, cb));
      const u32x2 ah1 = tr_read(khi, tr_offset(lane, kb0 + 4, cb));
      const u32x2 al0 = tr_read(klo, tr_offset(lane, kb0, cb));
      const u32x2 al1 = tr_read(klo, tr_offset(lane, kb0 + 4, cb));
      const u32x2 b0v = tr_read(vls, tr_offset(lane, kb0, eb));
      const u32x2 b1v = tr_read(vls, tr_offset(lane, kb0 + 4, eb));
      const u32x4 ah = {ah0.x, ah0.y, ah1.x, ah1.y};
      const u32x4 al = {al0.x, al0.y, al1.x, al1.y};
      const u32x4 bv = {b0v.x, b0v.y, b1v.x, b1v.y};
      acc = mfma32(as_bf16x8(ah), as_bf16x8(bv), acc);
      acc = mfma32(as_bf16x8(al), as_bf16x8(bv), acc);
    }
  }

  // partial S quarter: acc[v] = S[32cb + 8(v/4) + 4(lane/32) + v%4][32eb + lane%32]
  float* out = partial + ((int64_t)h * nchunks + chunk) * kStateFloats;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int c = 32 * cb + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
    const int e = 32 * eb + (lane & 31);
    out[c * kHeadDim + e] = acc[i];
  }
  // z: threads with the same tid%8 own the same 8 channels; fixed-order sum
#pragma unroll
  for (int i = 0; i < 8; ++i) zred[tid][i] = z8[i];
  __syncthreads();
  if (tid < kHeadDim) {
    const int cg = tid >> 3, ci = tid & 7;
    float zsum = 0.f;
    for (int t = cg; t < 256; t += 8) zsum += zred[t][ci];
    out[kHeadDim * kHeadDim + tid] = zsum;
  }
}

// Sums partials in chunk order, folds the affine map, writes the apply
// kernel's operands: for e-block eb, k-step s, lane l, element j:
// S'[16s + 8(l/32) + j][32eb + l%32], as bf16 hi and lo; then z (float32).
__global__ __launch_bounds__(256) void linear_reduce_kernel(const float* __restrict__ partial,
                                                            int32_t nchunks,
                                                            const float* __restrict__ aff_a,
                                                            const float* __restrict__ aff_b,
                                                            uint16_t* __restrict__ sop,
                                                            float* __restrict__ zout) {
  __shared__ float st[kStateFloats];
  const int h = blockIdx.x, tid = threadIdx.x;
  const float* ph = partial + (int64_t)h * nchunks * kStateFloats;
  for (int e = tid; e < kStateFloats; e += 256) {
    double s = 0.0;
    for (int c = 0; c < nchunks; ++c) s += (double)ph[(int64_t)c * kStateFloats + e];
    st[e] = (float)s;
  }
  __syncthreads();
  const float* z = st + kHeadDim * kHeadDim;
  // element index: ((eb * 4 + s) * 64 + lane) * 8 + j, hi half then lo half
  uint16_t* hi_out = sop + (int64_t)h * 2 * 4096;
  uint16_t* lo_out = hi_out + 4096;
  for (int idx = tid; idx < 4096; idx += 256) {
    const int j = idx & 7, lane = (idx >> 3) & 63, s = (idx >> 9) & 3, eb = idx >> 11;
    const int c = 16 * s + 8 * (lane >> 5) + j;
    const int e = 32 * eb + (lane & 31);
    const float a = aff_a ? aff_a[h * kHeadDim + e] : 1.f;
    const float b = aff_b ? aff_b[h * kHeadDim + e] : 0.f;
    const float val = a * st[c * kHeadDim + e] + z[c] * b;
    const uint32_t w = pack_bf16x2(val, val - bf16lo(pack_bf16x2(val, 0.f)));
    hi_out[idx] = (uint16_t)(w & 0xffffu);
    lo_out[idx] = (uint16_t)(w >> 16);
  }
  if (tid < kHeadDim) zout[h * kHeadDim + tid] = z[tid];
}

__global__ __launch_bounds__(256) void linear_apply_kernel(
    const uint16_t* __restrict__ q, int64_t nq, int64_t qst, int64_t qsh,
    const uint16_t* __restrict__ sop, const float* __restrict__ zin, int64_t tok_per_block,
    void* __restrict__ o, int64_t ost, int64_t osh, int32_t o_f32) {
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int h = blockIdx.y;
  const int hh = lane >> 5, qi = lane & 31;

  bf16x8 ahi[2][4], alo[2][4];
  const uint16_t* sh = sop + (int64_t)h * 2 * 4096;
#pragma unroll
  for (int eb = 0; eb < 2; ++eb)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int off = ((eb * 4 + s) * 64 + lane) * 8;
      ahi[eb][s] = as_bf16x8(*(const u32x4*)(sh + off));
      alo[eb][s] = as_bf16x8(*(const u32x4*)(sh + 4096 + off));
    }
  float zr[4][8];
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int j = 0; j < 8; ++j) zr[s][j] = zin[h * kHeadDim + 16 * s + 8 * hh + j];

  const int64_t b0 = (int64_t)blockIdx.x * tok_per_block;
  const int64_t b1 = std::min(nq, b0 + tok_per_block);
  for (int64_t base = b0 + 32 * wave; base < b1; base += 128) {
    const int64_t n = base + qi;
    const bool ok = n < b1;
    const uint16_t* qp = q + (int64_t)h * qsh + n * qst + 8 * hh;
    bf16x8 bhi[4], blo[4];
    float den = 0.f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (ok) w = *(const u32x4*)(qp + 16 * s);
      float f[8];
      f[0] = phi(bf16lo(w.x));
      f[1] = phi(bf16hi(w.x));
      f[2] = phi(bf16lo(w.y));
      f[3] = phi(bf16hi(w.y));
      f[4] = phi(bf16lo(w.z));
      f[5] = phi(bf16hi(w.z));
      f[6] = phi(bf16lo(w.w));
      f[7] = phi(bf16hi(w.w));
#pragma unroll
      for (int j = 0; j < 8; ++j) den = __builtin_fmaf(f[j], zr[s][j], den);
      u32x4 hi, lo;
      split8(f, hi, lo);
      bhi[s] = as_bf16x8(hi);
      blo[s] = as_bf16x8(lo);
    }
    den += __shfl_xor(den, 32, kWave);
    const float inv = 1.0f / den;
    f32x16 acc[2];
#pragma unroll
    for (int eb = 0; eb < 2; ++eb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[eb][i] = 0.f;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        acc[eb] = mfma32(ahi[eb][s], bhi[s], acc[eb]);
        acc[eb] = mfma32(ahi[eb][s], blo[s], acc[eb]);
        acc[eb] = mfma32(alo[eb][s], bhi[s], acc[eb]);
      }
    }
    if (!ok) continue;
    // acc[eb][4g + r] = O^T[32eb + 8g + 4hh + r][n]
    if (o_f32) {
      float* op = (float*)o + (int64_t)h * osh + n * ost + 4 * hh;
#pragma unroll
      for (int eb = 0; eb < 2; ++eb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 w = {acc[eb][4 * g] * inv, acc[eb][4 * g + 1] * inv, acc[eb][4 * g + 2] * inv,
                     acc[eb][4 * g + 3] * inv};
          *(f32x4*)(op + 32 * eb + 8 * g) = w;
        }
    } else {
      uint16_t* op = (uint16_t*)o + (int64_t)h * osh + n * ost + 4 * hh;
#pragma unroll
      for (int eb = 0; eb < 2; ++eb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          u32x2 w = {pack_bf16x2(acc[eb][4 * g] * inv, acc[eb][4 * g + 1] * inv),
                     pack_bf16x2(acc[eb][4 * g + 2] * inv, acc[eb][4 * g + 3] * inv)};
          *(u32x2*)(op + 32 * eb + 8 * g) = w;
        }
    }
  }
}

void state_chunking(int64_t nk, int32_t heads, int32_t& nchunks, int64_t& chunk_tok) {
  const int64_t blocks = std::max<int64_t>(1, (nk + kBlockTok - 1) / kBlockTok);
  int64_t want = std::max<int64_t>(1, (kTargetStateBlocks + heads - 1) / std::max(1, heads));
  want = std::min(want, blocks);
  chunk_tok = ((blocks + want - 1) / want) * kBlockTok;
  nchunks = (int32_t)((nk + chunk_tok - 1) / chunk_tok);
  if (nchunks < 1) nchunks = 1;
}

}  // namespace

size_t linear_workspace_bytes(int64_t n_kv, int32_t heads) {
  int32_t nchunks;
  int64_t chunk_tok;
  state_chunking(n_kv, heads, nchunks, chunk_tok);
  const size_t partial = (size_t)heads * nchunks * kStateFloats * sizeof(float);
  const size_t sop = (size_t)heads * 2 * 4096 * sizeof(uint16_t);
  const size_t z = (size_t)heads * kHeadDim * sizeof(float);
  return partial + sop + z;
}

hipError_t launch_linear(const uint16_t* q, int64_t nq, int64_t qst, int64_t qsh,
                         const uint16_t* k, const uint16_t* v, int64_t nk, int64_t kst,
                         int64_t ksh, int32_t heads, const float* aff_scale,
                         const float* aff_bias, void* o, int64_t ost, int64_t osh, bool o_f32,
                         void* ws, hipStream_t s) {
  if (heads == 0 || nq == 0) return hipSuccess;
  int32_t nchunks;
  int64_t chunk_tok;
  state_chunking(nk, heads, nchunks, chunk_tok);
  float* partial = (float*)ws;
  uint16_t* sop = (uint16_t*)(partial + (size_t)heads * nchunks * kStateFloats);
  float* z = (float*)(sop + (size_t)heads * 2 * 4096);
  hipLaunchKernelGGL(linear_state_kernel, dim3(nchunks, heads), dim3(256), 0, s, k, v, nk, kst,
                     ksh, chunk_tok, nchunks, partial);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(linear_reduce_kernel, dim3(heads), dim3(256), 0, s, partial, nchunks,
                     aff_scale, aff_bias, sop, z);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t per_block = 512;
  const int64_t nblocks = (nq + per_block - 1) / per_block;
  hipLaunchKernelGGL(linear_apply_kernel, dim3((unsigned)nblocks, heads), dim3(256), 0, s, q, nq,
                     qst, qsh, sop, z, per_block, o, ost, osh, o_f32 ? 1 : 0);
  return hipGetLastError();
}

}  // namespace zebra
