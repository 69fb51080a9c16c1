// elu+1 linear attention with the per-channel affine map (gfx950).
//
// Tolerant stages run linear(-centered) attention followed by a closed-form
// affine map (Zebra3D paper page, thelatestinai.com: Abstract; Table 3(a)).
// With phi(x) = elu(x) + 1:
//   S = sum_n phi(k_n) v_n^T,  z = sum_n phi(k_n),
//   out_m = a (*) (phi(q_m)^T S) / (phi(q_m)^T z) + b.
//
// Three kernels, streaming at HBM rate:
//  1. state: per (head, token chunk) partial S and z. K and V blocks of 64
//     tokens go to LDS row-major (the next block's loads in flight while one
//     is used); phi(K) is formed in float32 and split into bf16 hi + lo parts
//     (phi = hi + lo to ~2^-17), so two bf16 MFMAs give a float32-grade
//     product. The contraction runs over tokens, so both MFMA operands are
//     read token-transposed with ds_read_b64_tr_b16. Each of the 4 waves owns
//     one 32x32 quarter of S.
//  2. reduce: partial states summed over chunks in a fixed order (float64),
//     one thread per state element, into a float32 S and z per head.
//  3. apply: each workgroup folds the affine map into the state,
//     a (*) (phi^T S)/(phi^T z) + b = phi^T (S diag(a) + z b^T) / (phi^T z),
//     and keeps the folded state as bf16 hi/lo MFMA A-operands in registers;
//     then O^T = S'^T phi(Q)^T with three bf16 MFMAs per product (hi.hi,
//     hi.lo, lo.hi) and the float32 denominator phi(q).z, 32 queries per wave
//     and step, the next step's query loads in flight.
// No atomics: the result is bitwise reproducible.
#include <algorithm>

#include "common.h"

namespace zebra {

namespace {

typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr int kBlockTok = 64;
constexpr int kStateFloats = kHeadDim * kHeadDim + kHeadDim;  // S then z
// State workgroups per launch (all heads): one round of the 4 workgroups per
// CU the kernel's registers allow on 256 CUs. Measured at 512 views: 1,024
// ran 2.6% faster than 2,048 and faster than 768, 1,280 or 1,536 (a partial
// second round); the fp64 reduce sums the partials in chunk order either way.
constexpr int kTargetStateBlocks = 1024;

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
  // phi(K) hi and lo tiles, then (after the last block) the z reduction buffer
  __shared__ __attribute__((aligned(16))) uint8_t kt[2 * kBlockTok * 128];
  __shared__ __attribute__((aligned(16))) uint8_t vls[kBlockTok * 128];
  uint8_t* khi = kt;
  uint8_t* klo = kt + kBlockTok * 128;
  float(*zred)[9] = (float(*)[9])kt;
  static_assert(256 * 9 * sizeof(float) <= sizeof(kt), "z buffer fits");

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

  // this thread's two 16-byte pieces of a 64-token block: row e/8, chunk e%8;
  // the next block's loads are in flight while one block is used. K and V
  // are read once: non-temporal loads keep them from displacing L2 lines.
  u32x4 kn[2], vn[2];
  auto load_block = [&](int64_t b0) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int e = tid + 256 * u;
      const int64_t tok = b0 + (e >> 3);
      kn[u] = u32x4{0u, 0u, 0u, 0u};
      vn[u] = u32x4{0u, 0u, 0u, 0u};
      if (tok < t1) {
        kn[u] = __builtin_nontemporal_load((const u32x4*)(kh + tok * kst + 8 * (e & 7)));
        vn[u] = __builtin_nontemporal_load((const u32x4*)(vh + tok * kst + 8 * (e & 7)));
      }
    }
  };
  load_block(t0);
  for (int64_t b0 = t0; b0 < t1; b0 += kBlockTok) {
    const u32x4 kc[2] = {kn[0], kn[1]}, vc[2] = {vn[0], vn[1]};
    load_block(b0 + kBlockTok);
    __syncthreads();  // the previous block's LDS reads are done
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int e = tid + 256 * u;
      const int r = e >> 3, c = e & 7;
      const bool ok = b0 + r < t1;
      const u32x4 kw = kc[u];
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
      *(u32x4*)(vls + swz(r, c)) = vc[u];
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
  __syncthreads();  // the K tiles are no longer read
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

// Sums the partial states in chunk order (float64): one thread per element of
// [S | z], 8 chunks per round with their loads issued together.
__global__ __launch_bounds__(256) void linear_reduce_kernel(const float* __restrict__ partial,
                                                            int32_t nchunks,
                                                            float* __restrict__ state) {
  const int h = blockIdx.y;
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= kStateFloats) return;
  const float* ph = partial + (int64_t)h * nchunks * kStateFloats + e;
  double s = 0.0;
  int c = 0;
  for (; c + 8 <= nchunks; c += 8) {
    float x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = ph[(int64_t)(c + i) * kStateFloats];
#pragma unroll
    for (int i = 0; i < 8; ++i) s += (double)x[i];
  }
  for (; c < nchunks; ++c) s += (double)ph[(int64_t)c * kStateFloats];
  state[(int64_t)h * kStateFloats + e] = (float)s;
}

// phi of 8 bf16 channels (one 16-byte piece) -> hi/lo operands, and the
// partial denominator sum_j phi_j z_j
__device__ __forceinline__ void phi_split(u32x4 w, const float* zr, bf16x8& hi8, bf16x8& lo8,
                                          float& den) {
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
  for (int j = 0; j < 8; ++j) den = __builtin_fmaf(f[j], zr[j], den);
  u32x4 hi, lo;
  split8(f, hi, lo);
  hi8 = as_bf16x8(hi);
  lo8 = as_bf16x8(lo);
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void linear_apply_kernel(
    const uint16_t* __restrict__ q, int64_t nq, int64_t qst, int64_t qsh,
    const float* __restrict__ state, const float* __restrict__ aff_a,
    const float* __restrict__ aff_b, int64_t tok_per_block, void* __restrict__ o, int64_t ost,
    int64_t osh, int32_t o_f32) {
  // per wave: one 32-token x 128-byte tile, row-swizzled; queries come in and
  // bf16 outputs go out through it so that global accesses are whole rows
  __shared__ __attribute__((aligned(16))) uint8_t tile[4][32 * 128];
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int h = blockIdx.y;
  const int hh = lane >> 5, qi = lane & 31;
  uint8_t* tw = tile[wave];

  // A operands of O^T = S''^T phi(Q)^T, shared by the workgroup's waves in
  // LDS: for part p (0 hi, 1 lo), e-block eb, k-step s and lane l, the bf16
  // values S''[16s + 8(l/32) + j][32eb + l%32], j = 0..7
  __shared__ u32x4 aops[2][2][4][kWave];
  const float* st = state + (int64_t)h * kStateFloats;
  const float* z = st + kHeadDim * kHeadDim;
  {
    const int eb = wave >> 1, s0 = 2 * (wave & 1);  // each wave builds two k-steps
    const int e = 32 * eb + qi;
    const float a = aff_a ? aff_a[h * kHeadDim + e] : 1.f;
    const float b = aff_b ? aff_b[h * kHeadDim + e] : 0.f;
#pragma unroll
    for (int s = s0; s < s0 + 2; ++s) {
      float f[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int c = 16 * s + 8 * hh + j;
        f[j] = a * st[c * kHeadDim + e] + z[c] * b;
      }
      split8(f, aops[0][eb][s][lane], aops[1][eb][s][lane]);
    }
  }
  __shared__ __attribute__((aligned(16))) float zs[kHeadDim];
  if (tid < kHeadDim) zs[tid] = z[tid];
  __syncthreads();

  const int64_t b0 = (int64_t)blockIdx.x * tok_per_block;
  const int64_t b1 = std::min(nq, b0 + tok_per_block);
  const uint16_t* qh = q + (int64_t)h * qsh;
  const int lrow = lane >> 3, lch = lane & 7;  // row-major view: 8 rows per access
  // coalesced loads of a 32-token step: lane reads chunk lch of rows lrow + 8i;
  // the next step's loads are in flight while one step is used
  u32x4 qn[4];
  auto load_q = [&](int64_t base) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t n = base + 8 * i + lrow;
      qn[i] = u32x4{0u, 0u, 0u, 0u};
      if (n < b1) qn[i] = *(const u32x4*)(qh + n * qst + 8 * lch);
    }
  };
  load_q(b0 + 32 * wave);
  for (int64_t base = b0 + 32 * wave; base < b1; base += 128) {
    // queries -> LDS (row-major), then the operand layout: row qi, chunk 2s + hh
#pragma unroll
    for (int i = 0; i < 4; ++i) *(u32x4*)(tw + swz(8 * i + lrow, lch)) = qn[i];
    load_q(base + 128);
    u32x4 qc[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) qc[s] = *(const u32x4*)(tw + swz(qi, 2 * s + hh));
    const int64_t n = base + qi;
    bf16x8 bhi[4], blo[4];
    float den = 0.f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const f32x4 z0 = *(const f32x4*)(zs + 16 * s + 8 * hh);
      const f32x4 z1 = *(const f32x4*)(zs + 16 * s + 8 * hh + 4);
      const float zr[8] = {z0.x, z0.y, z0.z, z0.w, z1.x, z1.y, z1.z, z1.w};
      phi_split(qc[s], zr, bhi[s], blo[s], den);
    }
    den += __shfl_xor(den, 32, kWave);
    const float inv = 1.0f / den;
    // re-read the operands from LDS every step rather than keeping all 16 in
    // registers (the compiler would otherwise hoist the loop-invariant reads)
    asm volatile("" ::: "memory");
    // one e-block at a time: acc[4g + r] = O^T[32eb + 8g + 4hh + r][n]
#pragma unroll
    for (int eb = 0; eb < 2; ++eb) {
      f32x16 acc;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8 ahi = as_bf16x8(aops[0][eb][s][lane]);
        const bf16x8 alo = as_bf16x8(aops[1][eb][s][lane]);
        acc = mfma32(ahi, bhi[s], acc);
        acc = mfma32(ahi, blo[s], acc);
        acc = mfma32(alo, bhi[s], acc);
      }
      if (o_f32) {
        if (n < b1) {
          float* op = (float*)o + (int64_t)h * osh + n * ost + 32 * eb + 4 * hh;
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            f32x4 w = {acc[4 * g] * inv, acc[4 * g + 1] * inv, acc[4 * g + 2] * inv,
                       acc[4 * g + 3] * inv};
            *(f32x4*)(op + 8 * g) = w;
          }
        }
      } else {
        // bf16 rows through the tile: 8 bytes of row qi at channel 32eb + 8g + 4hh
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          u32x2 w = {pack_bf16x2(acc[4 * g] * inv, acc[4 * g + 1] * inv),
                     pack_bf16x2(acc[4 * g + 2] * inv, acc[4 * g + 3] * inv)};
          *(u32x2*)(tw + swz(qi, 4 * eb + g) + 8 * hh) = w;
        }
      }
    }
    if (!o_f32) {
      uint16_t* oh = (uint16_t*)o + (int64_t)h * osh;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 8 * i + lrow;
        const u32x4 w = *(const u32x4*)(tw + swz(r, lch));
        if (base + r < b1) *(u32x4*)(oh + (base + r) * ost + 8 * lch) = w;
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
  const size_t state = (size_t)heads * kStateFloats * sizeof(float);
  return partial + state;
}

hipError_t launch_linear_state(const uint16_t* k, const uint16_t* v, int64_t nk, int64_t kst,
                               int64_t ksh, int32_t heads, void* ws, float** state_out,
                               hipStream_t s) {
  int32_t nchunks;
  int64_t chunk_tok;
  state_chunking(nk, heads, nchunks, chunk_tok);
  float* partial = (float*)ws;
  float* state = partial + (size_t)heads * nchunks * kStateFloats;
  *state_out = state;
  hipLaunchKernelGGL(linear_state_kernel, dim3(nchunks, heads), dim3(256), 0, s, k, v, nk, kst,
                     ksh, chunk_tok, nchunks, partial);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(linear_reduce_kernel, dim3((kStateFloats + 255) / 256, heads), dim3(256), 0,
                     s, partial, nchunks, state);
  return hipGetLastError();
}

hipError_t launch_linear(const uint16_t* q, int64_t nq, int64_t qst, int64_t qsh,
                         const uint16_t* k, const uint16_t* v, int64_t nk, int64_t kst,
                         int64_t ksh, int32_t heads, const float* aff_scale,
                         const float* aff_bias, void* o, int64_t ost, int64_t osh, bool o_f32,
                         void* ws, hipStream_t s) {
  if (heads == 0 || nq == 0) return hipSuccess;
  float* state = nullptr;
  hipError_t err = launch_linear_state(k, v, nk, kst, ksh, heads, ws, &state, s);
  if (err != hipSuccess) return err;
  // about 32,768 workgroups of 4 waves over all heads (8 rounds of the 4 per CU
  // the registers allow); each wave loops over 32-query steps with the next
  // step's loads in flight. Measured at 512 views against 4,096 workgroups:
  // 8,192 -2.3%, 16,384 -5%, 32,768 -6.4%, one 128-query step each (88k) +2.5%.
  const int64_t per_block =
      std::max<int64_t>(128, ((nq * heads + 32767) / 32768 + 127) / 128 * 128);
  const int64_t nblocks = (nq + per_block - 1) / per_block;
  hipLaunchKernelGGL(linear_apply_kernel, dim3((unsigned)nblocks, heads), dim3(256), 0, s, q, nq,
                     qst, qsh, state, aff_scale, aff_bias, per_block, o, ost, osh, o_f32 ? 1 : 0);
  return hipGetLastError();
}

}  // namespace zebra
