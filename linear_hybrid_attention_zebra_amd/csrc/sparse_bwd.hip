// Backward pass of tile-sparse attention with landmarks (gfx950).
//
// For the optional refinement of a converted model (Zebra3D paper page,
// Tables 18-19): the gradients of sum(dout * out) for one tile-sparse stage,
// the selection held fixed. Per query row with columns c (kept tokens, then
// one landmark per omitted tile; Figure 1 caption) and P = softmax:
//   dP_c = dout . v_c,  D = dout . out,  dS_c = P_c (dP_c - D),
//   dq = scale sum_c dS_c k_c,  dk_c = scale dS_c q,  dv_c = P_c dout.
// A landmark's key and value are the means of its tile, so every token of
// tile j receives 1/n_j of the landmark's dk and dv.
//
// Steps (the forward runs first, writing the log2 softmax normaliser lse of
// every query, so P_c = 2^(c s_c + bias_c - lse); dout enters the products
// in bf16):
//  1. the kept-tile bit matrix [H][Tq][Tk/32] and, by a stable counting sort
//     over it, for every key tile the ascending list of query tiles keeping it;
//  2. dq: one workgroup per (head, query tile), over its kept tiles and
//     landmark blocks: dS and dq, with D = dout . out from the forward's
//     float32 output (formed while dout is packed). With only the normaliser
//     of an earlier forward at hand, a first sweep forms D = sum_c P_c dP_c
//     from the same float32 P and dP and renormalises lse by sum_c P_c. D
//     from a bf16-rounded output would be off by about 2^-9 |dout| |out|,
//     which dP - D amplifies where the attention is concentrated;
//  3. dk, dv of the landmark rows: one workgroup per (head, block of KT
//     landmark rows), over every query tile, the kept tiles masked;
//  4. dk, dv of the key tiles: one workgroup per (head, key tile), over the
//     query tiles keeping it, plus the tile's landmark share from step 3.
// Steps 2-4 run as a sequence of launches over chunks (key tiles for dq,
// query tiles for dk and dv) so that the workgroups running together share
// one chunk's operands in L2; each launch adds into float32 accumulators,
// in launch order.
// Steps 2 and 4 stage their blocks global -> LDS directly into two-stage
// rings (step 4 only while the rings leave two waves per SIMD): one block
// ahead behind a barrier per step, or, for dq with 64-query and 64-key tiles
// (the key-half layout, where each wave stages only its own rows), two blocks
// ahead with no barrier.
// Steps 2-4 recompute S and dP with bf16 MFMA 32x32x16 and accumulate in
// float32; dS enters its products as a bf16 pair (float32-grade), P as bf16
// (as in the forward). Sums run in a fixed order: no atomics in any
// floating-point sum, so the gradients are bitwise reproducible.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "common.h"

namespace zebra {

namespace {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;

constexpr float kLog2eB = 1.4426950408889634f;

// 16-byte chunk `chunk` of 128-byte row `row`, XOR swizzled as in the forward
__device__ __forceinline__ int swz_f(int row) { return (((row >> 1) & 1) << 2) | ((row >> 2) & 3); }
__device__ __forceinline__ uint32_t swz(int row, int chunk) {
  return (uint32_t)(row * 128 + ((chunk ^ swz_f(row)) << 4));
}

// 8 channels of a bf16 or float32 row as bf16 (round to nearest even)
__device__ __forceinline__ u32x4 load8_bf16(const void* base, int64_t elem, bool f32) {
  if (!f32) return *(const u32x4*)((const uint16_t*)base + elem);
  const f32x4 a = *(const f32x4*)((const float*)base + elem);
  const f32x4 b = *(const f32x4*)((const float*)base + elem + 4);
  return u32x4{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]),
               pack_bf16x2(b[2], b[3])};
}

// Operand of a 32x32x16 MFMA whose contraction runs over the rows of an LDS
// tile (rows x 64 channels, swizzled): lane l holds, for channel
// 32 db + 16 (G % 2) + 4 (S % 4) + {0..3} (G = l / 16, S = l % 16), the 8 rows
// 16 m + 4 (G / 2) + S / 4 + {0, 8} ... in the order that matches the
// C-layout of a 32x32 score block (the forward's V^T read).
__device__ __forceinline__ bf16x8 tr_operand(const lds_u8* tile, int m, int db, int lane) {
  const int G = lane >> 4, S = lane & 15;
  const int col = 32 * db + 16 * (G & 1) + 4 * (S & 3);
  const int chunk = col >> 3, half = (col & 7) ? 8 : 0;
  const int r0 = 16 * m + 4 * (G >> 1) + (S >> 2);
  const i16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(tile + swz(r0, chunk) + half));
  const i16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(tile + swz(r0 + 8, chunk) + half));
  const u32x2 w0 = __builtin_bit_cast(u32x2, t0), w1 = __builtin_bit_cast(u32x2, t1);
  return as_bf16x8(u32x4{w0.x, w0.y, w1.x, w1.y});
}

// Row operand: lane l holds channels 16 s + 8 (l / 32) .. +7 of tile row `row`
__device__ __forceinline__ bf16x8 row_operand(const lds_u8* tile, int row, int s, int hh) {
  return as_bf16x8(*(const __attribute__((address_space(3))) u32x4*)(tile + swz(row, 2 * s + hh)));
}

// 16 scores of one 32x32 C-layout block -> two bf16 operands (16 rows each)
__device__ __forceinline__ void pack16(const float* x, bf16x8& lo8, bf16x8& hi8) {
  uint32_t w[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
  lo8 = as_bf16x8(u32x4{w[0], w[1], w[2], w[3]});
  hi8 = as_bf16x8(u32x4{w[4], w[5], w[6], w[7]});
}

// The same, float32-grade: x = big + small with both parts bf16 (x - big is
// exact in float32 and rounds to within 2^-17 of x), so two MFMAs give the
// product to float32 accuracy. dS = P (dP - D) cancels, which bf16 alone
// would amplify.
__device__ __forceinline__ void pack16_split(const float* x, bf16x8& lo8, bf16x8& hi8,
                                             bf16x8& lo8s, bf16x8& hi8s) {
  uint32_t w[8], r[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    w[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
    r[i] = pack_bf16x2(x[2 * i] - bf16lo(w[i]), x[2 * i + 1] - bf16hi(w[i]));
  }
  lo8 = as_bf16x8(u32x4{w[0], w[1], w[2], w[3]});
  hi8 = as_bf16x8(u32x4{w[4], w[5], w[6], w[7]});
  lo8s = as_bf16x8(u32x4{r[0], r[1], r[2], r[3]});
  hi8s = as_bf16x8(u32x4{r[4], r[5], r[6], r[7]});
}

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* kbar_b;  // bf16 landmark rows [H][tk][64], or null without landmarks
  const uint16_t* vbar_b;
  const int32_t* sel;      // [H][tq][top_k]
  const void* dout;
  const uint16_t* dout_b;  // dout packed as bf16 [H][nq][64]
  void* dq;
  void* dk;
  void* dv;
  int64_t nq, qst, qsh;
  int64_t nk, kst, ksh;
  int64_t dst, dsh;        // dout strides
  int64_t qgst, qgsh;      // dq strides
  int64_t kgst, kgsh;      // dk, dv strides
  int32_t heads, tq, tk, top_k, bit_words;
  float c;                 // scale * log2(e)
  float scale;
  int32_t g_f32, landmarks, log_count;
  float lm_log2_kt, lm_tail_corr;  // log-count biases (log2 units; tail in score units)
  float* lse;              // [H][nq]; dq sweep 0 (when run) renormalises it in place
  float* dsum;             // D [H][nq]: from the float32 output, or by dq sweep 0
  const uint32_t* bits;    // [H][tq][bit_words] kept tiles
  const int32_t* list_off; // [H][tk + 1]
  const int32_t* list;     // [H][tq * top_k] query tiles keeping each key tile
  float* dkbar;            // [H][tk][64] float32 landmark gradients (accumulated per launch)
  float* dvbar;
  // chunked launches: this launch covers query tiles [q_lo, q_hi) (dk, dv) or
  // key tiles [k_lo, k_hi) (dq); contributions add up in launch order
  int32_t q_lo, q_hi, k_lo, k_hi, first, last;
  float* acc_k;            // [H][nk][64] float32 dk, dv accumulators
  float* acc_v;
  float* l_acc;            // [H][nq] sum of P', sum of P' dP (dq sweep 0)
  float* d_acc;
  float* dq_acc;           // [H][nq][64] float32 dq accumulator (dq sweep 1)
  // phased walks (dq, and dk/dv of key tiles): 0, or the workgroups the
  // device runs at once; an item then starts its walk of this launch's range
  // at the first entry at or after position (item mod P) / P and wraps around,
  // so the items in flight walk the same part of the range together (as in
  // the forward's split keys). The walk order changes only summation order.
  int64_t phase_period;
};

// The lanes of a 32x32 C-layout block whose row (key) is set in a uniform
// 32-bit column mask, for the register whose rows are off + 4 hh (hh = lane
// half): a 64-bit lane mask of two sign-extended bits, built with scalar ops.
__device__ __forceinline__ uint64_t half_lanes(uint32_t w, int off) {
  const uint32_t lo = (uint32_t)(((int32_t)(w << (31 - off))) >> 31);
  const uint32_t hi = (uint32_t)(((int32_t)(w << (27 - off))) >> 31);
  return ((uint64_t)hi << 32) | lo;
}

// 16 bytes per lane global -> LDS directly (the lane's bytes land at
// dst + 16 lane)
// 16 bytes per lane from a buffer resource straight into LDS (the lane's
// bytes land at dst + 16 lane); reads past the resource's records return zeros
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ void b2l16(__amdgpu_buffer_rsrc_t r, void* dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16,
                                           voff, 0, 0, 0);
}
__device__ __forceinline__ void g2l16(const void* src, void* dst) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
}

// 4 bytes per lane global -> LDS directly (the lane's word lands at dst + 4 lane)
__device__ __forceinline__ void g2l4(const void* src, void* dst) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 4, 0, 0);
}

// Read-only index data (kept lists, bits) read as constant memory by the
// key-half dq kernel: nothing writes it while the kernel runs, so uniform reads
// become scalar loads, which the vector-memory counter that its steps wait on
// does not count (a vector load there would make a step wait for its own
// prefetch).
typedef const __attribute__((address_space(4))) int32_t* cint_p;
typedef const __attribute__((address_space(4))) uint32_t* cuint_p;

// first index in [lo, hi) of the ascending array a with a[i] >= x
__device__ __forceinline__ int lower_bound_i32(const int32_t* a, int lo, int hi, int x) {
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] < x) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

// ---------------------------------------------------------------------------
// 2. kept-tile bits, per-key-tile counts, offsets, ordered lists
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_fill_u32_kernel(uint32_t* __restrict__ p, int64_t n) {
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256)
    p[e] = 0u;
}

// dout (bf16 or float32, any token/head strides) -> packed bf16 [H][nq][64],
// 8 channels per thread; the dk, dv kernels stage it global -> LDS directly
// With the forward's float32 output o given, the same pass also forms
// D = dout . o per query (dout rounded to bf16, as the dP products see it):
// the eight lanes of a row each take 8 channels, then add in a fixed tree.
__global__ __launch_bounds__(256) void bwd_pack_dout_kernel(const void* __restrict__ dout,
                                                            int64_t dst, int64_t dsh, int32_t f32,
                                                            int64_t nq, int64_t n_pieces,
                                                            uint16_t* __restrict__ out,
                                                            const float* __restrict__ o,
                                                            int64_t ost, int64_t osh,
                                                            float* __restrict__ dsum) {
  // n_pieces is 8 per row and the stride a multiple of 256, so the eight
  // lanes of a row are in one wave and take the loop together
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n_pieces;
       e += (int64_t)gridDim.x * 256) {
    const int64_t rowi = e >> 3, c8 = e & 7;
    const int64_t h = rowi / nq, q = rowi - h * nq;
    const u32x4 w = load8_bf16(dout, h * dsh + q * dst + 8 * c8, f32 != 0);
    *(u32x4*)(out + rowi * kHeadDim + 8 * c8) = w;
    if (o != nullptr) {
      const float* orow = o + h * osh + q * ost + 8 * c8;
      const f32x4 a = *(const f32x4*)orow, b = *(const f32x4*)(orow + 4);
      float d = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4& x = i < 2 ? a : b;
        const int j = 2 * (i & 1);
        d = __builtin_fmaf(__uint_as_float(w[i] << 16), x[j], d);
        d = __builtin_fmaf(__uint_as_float(w[i] & 0xffff0000u), x[j + 1], d);
      }
      d += __shfl_xor(d, 1);
      d += __shfl_xor(d, 2);
      d += __shfl_xor(d, 4);
      if (c8 == 0) dsum[rowi] = d;
    }
  }
}

// Kept-tile bit matrix and per-key-tile counts. One workgroup per (head,
// rows_per_wg query tiles, at most kBitsRows): each row's bits are set in LDS and stored whole, and the
// counts of the workgroup's rows gather in an LDS histogram that is added to
// the global counts once (integer sums, so the result does not depend on
// the order). Dynamic LDS: tk counters, then bit_words words.
constexpr int kBitsRows = 64;
__global__ __launch_bounds__(256) void bwd_bits_kernel(const int32_t* __restrict__ sel,
                                                       int32_t tq, int32_t tk, int32_t top_k,
                                                       int32_t bit_words, int32_t rows_per_wg,
                                                       uint32_t* __restrict__ bits,
                                                       int32_t* __restrict__ count) {
  extern __shared__ uint32_t bits_lds[];
  uint32_t* cnt = bits_lds;
  uint32_t* wb = bits_lds + tk;
  const int tid = threadIdx.x;
  const int h = blockIdx.y;
  const int i0 = blockIdx.x * rows_per_wg, i1 = min(tq, i0 + rows_per_wg);
  for (int j = tid; j < tk; j += 256) cnt[j] = 0u;
  for (int i = i0; i < i1; ++i) {
    const int64_t row = (int64_t)h * tq + i;
    for (int e = tid; e < bit_words; e += 256) wb[e] = 0u;
    __syncthreads();  // (also: the histogram is cleared)
    for (int e = tid; e < top_k; e += 256) {
      const int j = min(max(sel[row * top_k + e], 0), tk - 1);
      atomicOr(&wb[j >> 5], 1u << (j & 31));
      atomicAdd(&cnt[j], 1u);
    }
    __syncthreads();
    for (int e = tid; e < bit_words; e += 256) bits[row * bit_words + e] = wb[e];
    __syncthreads();  // the row is stored before the next one clears it
  }
  for (int j = tid; j < tk; j += 256)
    if (cnt[j] != 0u) atomicAdd(&count[(int64_t)h * tk + j], (int)cnt[j]);
}

// exclusive scan of the counts of one head -> list offsets (head h starts at
// h * tq * top_k); off has tk + 1 entries per head
__global__ __launch_bounds__(256) void bwd_scan_kernel(const int32_t* __restrict__ count,
                                                       int32_t tk, int64_t per_head,
                                                       int32_t* __restrict__ off) {
  __shared__ int32_t part[256];
  const int h = blockIdx.x, t = threadIdx.x;
  const int per = (tk + 255) / 256;
  const int j0 = min(tk, t * per), j1 = min(tk, j0 + per);
  int s = 0;
  for (int j = j0; j < j1; ++j) s += count[(int64_t)h * tk + j];
  part[t] = s;
  __syncthreads();
  if (t == 0) {
    int run = 0;
    for (int i = 0; i < 256; ++i) {
      const int x = part[i];
      part[i] = run;
      run += x;
    }
  }
  __syncthreads();
  int64_t run = (int64_t)h * per_head + part[t];
  int32_t* oh = off + (int64_t)h * (tk + 1);
  for (int j = j0; j < j1; ++j) {
    oh[j] = (int32_t)run;
    run += count[(int64_t)h * tk + j];
  }
  if (t == 255) oh[tk] = (int32_t)run;  // end of the head's last list
}

// one workgroup of 64 threads per (head, bit word): thread t owns a contiguous
// range of query tiles; two passes give every key tile of the word its query
// tiles in ascending order
__global__ __launch_bounds__(64) void bwd_list_kernel(const uint32_t* __restrict__ bits,
                                                      int32_t tq, int32_t tk, int32_t bit_words,
                                                      const int32_t* __restrict__ off,
                                                      int32_t* __restrict__ list) {
  __shared__ int32_t cnt[64][33];
  const int w = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
  const int per = (tq + 63) / 64;
  const int i0 = min(tq, t * per), i1 = min(tq, i0 + per);
  const uint32_t* bh = bits + (int64_t)h * tq * bit_words + w;
  int c[32];
#pragma unroll
  for (int b = 0; b < 32; ++b) c[b] = 0;
  for (int i = i0; i < i1; ++i) {
    const uint32_t word = bh[(int64_t)i * bit_words];
#pragma unroll
    for (int b = 0; b < 32; ++b) c[b] += (word >> b) & 1u;
  }
#pragma unroll
  for (int b = 0; b < 32; ++b) cnt[t][b] = c[b];
  __syncthreads();
  if (t < 32) {  // exclusive scan over threads for bit t
    int run = 0;
    for (int i = 0; i < 64; ++i) {
      const int x = cnt[i][t];
      cnt[i][t] = run;
      run += x;
    }
  }
  __syncthreads();
  const int32_t* oh = off + (int64_t)h * (tk + 1);
#pragma unroll
  for (int b = 0; b < 32; ++b) {
    const int j = 32 * w + b;
    c[b] = j < tk ? oh[j] + cnt[t][b] : 0;
  }
  for (int i = i0; i < i1; ++i) {
    const uint32_t word = bh[(int64_t)i * bit_words];
#pragma unroll
    for (int b = 0; b < 32; ++b)
      if ((word >> b) & 1u) list[c[b]++] = i;
  }
}

// ---------------------------------------------------------------------------
// 3-4. dk, dv: one workgroup per (head, column block); wave w owns 32 columns
// ---------------------------------------------------------------------------
template <int QT, int KT, bool LM>
__global__ __launch_bounds__(KT * 2) __attribute__((amdgpu_waves_per_eu(2))) void bwd_dkdv_kernel(BwdParams p) {
  constexpr int W = KT / 32;
  constexpr int QC = QT / 32;  // 32-query chunks per query tile
  constexpr int KB = QT * 128 / 1024;  // 1 KB pieces per Q (or dout) tile
  constexpr int NU = KB / W;           // pieces per wave per tensor
  static_assert(KB % W == 0, "load split");
  // Two-stage rings of the query side (Q, dout, lse, D), loaded global -> LDS
  // directly one query tile ahead; distinct arrays per stage (see the dq kernel).
  __shared__ u32x4 qs0[QT * 8], ds0[QT * 8], qs1[QT * 8], ds1[QT * 8];
  __shared__ float lse0[QT], dsm0[QT], lse1[QT], dsm1[QT];
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int hh = lane >> 5, kl = lane & 31;
  const int n_blocks = LM ? (p.tk + KT - 1) / KT : p.tk;
  const int h = blockIdx.y;
  const int lrow = lane >> 3;
  const bool gf = p.g_f32 != 0;
  // byte offsets of the lane's 16 bytes of piece v within a staged query tile:
  // Q rows p.qst elements apart, packed dout rows 64
  uint32_t off_q[NU], off_d[NU];
#pragma unroll
  for (int v = 0; v < NU; ++v) {
    const int r = 8 * (wave + W * v) + lrow;
    const uint32_t c16 = 16u * (uint32_t)((lane & 7) ^ swz_f(r));
    off_q[v] = (uint32_t)r * (uint32_t)p.qst * 2u + c16;
    off_d[v] = (uint32_t)r * (uint32_t)kHeadDim * 2u + c16;
  }
  // per-lane operand read offsets within a staged tile (see the dq kernel):
  // row operands of row kl (+ 32 per query chunk), transposed operands at
  // rows r0 and r0 + 8 (+ 16 per 16-query step) of channel block db
  uint32_t roff[4], toff[2][2];
#pragma unroll
  for (int s = 0; s < 4; ++s) roff[s] = swz(kl, 2 * s + hh);
  {
    const int G = lane >> 4, S = lane & 15;
    const int r0 = 4 * (G >> 1) + (S >> 2);
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      const int col = 32 * db + 16 * (G & 1) + 4 * (S & 3);
      const int chunk = col >> 3, half = (col & 7) ? 8 : 0;
      toff[db][0] = swz(r0, chunk) + half;
      toff[db][1] = swz(r0 + 8, chunk) + half;
    }
  }
  auto row_op = [&](const lds_u8* tile, int qc, int s) -> bf16x8 {
    return as_bf16x8(*(const __attribute__((address_space(3))) u32x4*)(tile + roff[s] + 4096 * qc));
  };
  auto tr_op = [&](const lds_u8* tile, int m, int db) -> bf16x8 {
    const i16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(tile + toff[db][0] + 2048 * m));
    const i16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(tile + toff[db][1] + 2048 * m));
    const u32x2 w0 = __builtin_bit_cast(u32x2, t0), w1 = __builtin_bit_cast(u32x2, t1);
    return as_bf16x8(u32x4{w0.x, w0.y, w1.x, w1.y});
  };
  for (int cb = blockIdx.x; cb < n_blocks; cb += gridDim.x) {
    // this lane's column (key token or landmark row) and its validity
    const int col = KT * cb + 32 * wave + kl;
    int rows_valid;  // valid columns of the block
    const uint16_t* kb;
    const uint16_t* vb;
    int64_t kstride;
    if constexpr (LM) {
      rows_valid = min(KT, p.tk - KT * cb);
      kb = p.kbar_b + (int64_t)h * p.tk * kHeadDim;
      vb = p.vbar_b + (int64_t)h * p.tk * kHeadDim;
      kstride = kHeadDim;
    } else {
      rows_valid = (int)min<int64_t>(KT, p.nk - (int64_t)KT * cb);
      kb = p.k + (int64_t)h * p.ksh;
      vb = p.v + (int64_t)h * p.ksh;
      kstride = p.kst;
    }
    const int lcol = 32 * wave + kl;  // column within the block
    const bool cvalid = lcol < rows_valid;
    // B operands K^T and V^T of this lane's column: channels 16 s + 8 hh .. +7
    bf16x8 kop[4], vop[4];
    {
      const int64_t row = (int64_t)KT * cb + (cvalid ? lcol : 0);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
        if (cvalid) {
          a = *(const u32x4*)(kb + row * kstride + 16 * s + 8 * hh);
          b = *(const u32x4*)(vb + row * kstride + 16 * s + 8 * hh);
        }
        kop[s] = as_bf16x8(a);
        vop[s] = as_bf16x8(b);
      }
    }
    // logit bias of the column in log2 units (landmarks under the log count)
    float bias = 0.f;
    if constexpr (LM) {
      if (p.log_count) {
        bias = p.lm_log2_kt;
        const int64_t tail = p.nk - (int64_t)(p.tk - 1) * KT;
        if (col == p.tk - 1 && tail < KT) bias += p.lm_tail_corr * p.c;
      }
    }
    f32x16 dkacc[2], dvacc[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      dkacc[0][i] = 0.f;
      dkacc[1][i] = 0.f;
      dvacc[0][i] = 0.f;
      dvacc[1][i] = 0.f;
    }
    int n_i, i_base;
    if constexpr (LM) {
      n_i = p.q_hi - p.q_lo;
      i_base = p.q_lo;
    } else {  // the part of the (ascending) list inside [q_lo, q_hi)
      const int32_t* oh = p.list_off + (int64_t)h * (p.tk + 1);
      const int b0 = oh[cb], b1 = oh[cb + 1];
      i_base = lower_bound_i32(p.list, b0, b1, p.q_lo);
      n_i = lower_bound_i32(p.list, i_base, b1, p.q_hi) - i_base;
    }
    if (n_i == 0 && !p.first && !p.last) continue;  // nothing to add in this launch
    // query tile of list entry ii (a selection with repeated entries would
    // leave list slots unwritten)
    int rot = 0;  // phased walk of the query tiles keeping this key tile
    if constexpr (!LM) {
      if (p.phase_period > 0 && n_i > 1) {
        const int64_t idx = (int64_t)h * gridDim.x + cb;  // dispatch order: x, then y
        const int target =
            p.q_lo + (int)((idx % p.phase_period) * (p.q_hi - p.q_lo) / p.phase_period);
        const int r = lower_bound_i32(p.list, i_base, i_base + n_i, target) - i_base;
        rot = r < n_i ? r : 0;
      }
    }
    auto qtile_of = [&](int ii) -> int {
      if constexpr (LM) return i_base + ii;
      const int jj = ii + rot < n_i ? ii + rot : ii + rot - n_i;
      return min(max(p.list[i_base + jj], 0), p.tq - 1);
    };
    // stage query tile qt through buffer resources whose records end at the
    // tile's last valid row (rows past nq read as zeros; they are masked below)
    auto issue = [&](int qt, auto stc) {
      constexpr bool kS1 = decltype(stc)::value == 1;
      u32x4* qd = kS1 ? qs1 : qs0;
      u32x4* dd = kS1 ? ds1 : ds0;
      const int64_t last = p.nq - 1;
      const int64_t q0 = (int64_t)qt * QT;
      const int rows = (int)min<int64_t>(QT, p.nq - q0);
      const __amdgpu_buffer_rsrc_t rq = rows_rsrc(
          p.q + (int64_t)h * p.qsh + q0 * p.qst,
          (uint32_t)(((int64_t)(rows - 1) * p.qst + kHeadDim) * 2));
      const __amdgpu_buffer_rsrc_t rd = rows_rsrc(
          p.dout_b + ((int64_t)h * p.nq + q0) * kHeadDim, (uint32_t)rows * kHeadDim * 2u);
#pragma unroll
      for (int v = 0; v < NU; ++v) {
        const int u = wave + W * v;
        b2l16(rq, &qd[64 * u], off_q[v]);
        b2l16(rd, &dd[64 * u], off_d[v]);
      }
      // lse and D of the tile's rows, 4 bytes per lane in pieces of 64 rows:
      // piece j holds rows 64 (j / 2).. of lse (j even) or D (j odd)
      constexpr int NL = QT >= 64 ? QT / 64 : 1;
#pragma unroll
      for (int j = wave; j < 2 * NL; j += W) {
        const int r = 64 * (j >> 1) + lane;
        if (r < QT) {
          const int64_t qr = min((int64_t)qt * QT + r, last);
          const float* src = ((j & 1) ? p.dsum : p.lse) + (int64_t)h * p.nq + qr;
          float* dst = (j & 1) ? (kS1 ? dsm1 : dsm0) : (kS1 ? lse1 : lse0);
          g2l4(src, dst + 64 * (j >> 1));
        }
      }
    };
    auto step = [&](int ii, auto stc) {
      constexpr bool kS1 = decltype(stc)::value == 1;
      __syncthreads();  // tile ii has landed for every wave; the other stage is free
      if (ii + 1 < n_i) {
        if constexpr (kS1)
          issue(qtile_of(ii + 1), S0{});
        else
          issue(qtile_of(ii + 1), S1{});
      }
      __builtin_amdgcn_sched_barrier(0);  // (keeps the load addressing out of the products)
      const lds_u8* qtile = (const lds_u8*)(kS1 ? qs1 : qs0);
      const lds_u8* dtile = (const lds_u8*)(kS1 ? ds1 : ds0);
      const float* lse_s = kS1 ? lse1 : lse0;
      const float* dsum_s = kS1 ? dsm1 : dsm0;
      const int qt = qtile_of(ii);
      // rows of the tile past nq (only the last query tile): excluded
      const int64_t vr = p.nq - (int64_t)qt * QT;
      // kept mask of this lane's landmark column for query tile qt
      bool masked = !cvalid;
      if constexpr (LM) {
        const int wi = (KT * cb + 32 * wave) / 32;  // the word of this wave's 32 columns
        const uint32_t word =
            wi < p.bit_words ? p.bits[((int64_t)h * p.tq + qt) * p.bit_words + wi] : 0u;
        masked = masked || ((word >> kl) & 1u);
      }
      // an excluded landmark column enters with logit bias -inf (probability
      // zero); key tile columns past the end need no exclusion: a lane adds
      // only into its own column's dk and dv, which are never stored
      const float cbias = masked ? -INFINITY : bias;
#pragma unroll
      for (int qc = 0; qc < QC; ++qc) {
        // S = Q K^T and dP = dout V^T for 32 queries x this wave's 32 columns:
        // lane = column, register v = query 32 qc + 8 (v / 4) + 4 hh + v % 4
        f32x16 sacc, pacc;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const bf16x8 aq = row_op(qtile, qc, s);
          const bf16x8 ad = row_op(dtile, qc, s);
          if (s == 0) {
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, kop[0], f32x16{}, 0, 0, 0);
            pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ad, vop[0], f32x16{}, 0, 0, 0);
          } else {
            sacc = mfma32(aq, kop[s], sacc);
            pacc = mfma32(ad, vop[s], pacc);
          }
        }
        // excluded query rows of this chunk as -inf scores
        const int64_t vq = vr - 32 * qc;  // valid rows of the chunk
        const uint32_t w = vq >= 32 ? 0u : (vq <= 0 ? ~0u : ~0u << vq);
        if (w != 0u) {
#pragma unroll
          for (int v = 0; v < 16; ++v)
            if (__builtin_amdgcn_inverse_ballot_w64(half_lanes(w, 8 * (v >> 2) + (v & 3))))
              sacc[v] = -INFINITY;
        }
        float pr[16], dsr[16];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int q0 = 32 * qc + 8 * g + 4 * hh;
          const f32x4 l4 = *(const __attribute__((address_space(3))) f32x4*)&lse_s[q0];
          const f32x4 d4 = *(const __attribute__((address_space(3))) f32x4*)&dsum_s[q0];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = 4 * g + r;
            const float pv =
                LM ? __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[i], p.c, cbias) - l4[r])
                   : __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[i], p.c, -l4[r]));
            pr[i] = pv;
            dsr[i] = pv * (pacc[i] - d4[r]);
          }
        }
        bf16x8 plo, phi, slo, shi, slo2, shi2;
        pack16(pr, plo, phi);
        pack16_split(dsr, slo, shi, slo2, shi2);
        // dV += P^T dout, dK += dS^T Q over these 32 queries (two 16-query chunks)
#pragma unroll
        for (int db = 0; db < 2; ++db) {
          const bf16x8 d0 = tr_op(dtile, 2 * qc, db);
          const bf16x8 d1 = tr_op(dtile, 2 * qc + 1, db);
          const bf16x8 q0 = tr_op(qtile, 2 * qc, db);
          const bf16x8 q1 = tr_op(qtile, 2 * qc + 1, db);
          dvacc[db] = mfma32(plo, d0, dvacc[db]);
          dvacc[db] = mfma32(phi, d1, dvacc[db]);
          dkacc[db] = mfma32(slo, q0, dkacc[db]);
          dkacc[db] = mfma32(shi, q1, dkacc[db]);
          dkacc[db] = mfma32(slo2, q0, dkacc[db]);
          dkacc[db] = mfma32(shi2, q1, dkacc[db]);
        }
      }
    };
    __syncthreads();  // every wave is done with the previous block's rings
    if (n_i > 0) issue(qtile_of(0), S0{});
    {
      int ii = 0;
      for (; ii + 2 <= n_i; ii += 2) {
        step(ii, S0{});
        step(ii + 1, S1{});
      }
      if (ii < n_i) step(ii, S0{});
    }
    // epilogue: lane holds channel 32 db + kl of rows (columns of the block)
    // 32 wave + 8 (v / 4) + 4 hh + v % 4
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      const int ch = 32 * db + kl;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int lc = 32 * wave + 8 * (v >> 2) + 4 * hh + (v & 3);
        if (lc >= rows_valid) continue;
        const int64_t row = (int64_t)KT * cb + lc;
        float gk = p.scale * dkacc[db][v];
        float gv = dvacc[db][v];
        float* ak = LM ? p.dkbar : p.acc_k;
        float* av = LM ? p.dvbar : p.acc_v;
        const int64_t ai = ((int64_t)h * (LM ? p.tk : p.nk) + row) * kHeadDim + ch;
        if (!p.first) {  // add this launch's query tiles to the earlier ones
          gk += ak[ai];
          gv += av[ai];
        }
        if (LM || !p.last) {
          ak[ai] = gk;
          av[ai] = gv;
        } else {
          if (p.landmarks && p.dkbar != nullptr) {  // this tile's landmark share
            const float inv_n = 1.0f / (float)rows_valid;
            gk += p.dkbar[((int64_t)h * p.tk + cb) * kHeadDim + ch] * inv_n;
            gv += p.dvbar[((int64_t)h * p.tk + cb) * kHeadDim + ch] * inv_n;
          }
          if (gf) {
            ((float*)p.dk)[(int64_t)h * p.kgsh + row * p.kgst + ch] = gk;
            ((float*)p.dv)[(int64_t)h * p.kgsh + row * p.kgst + ch] = gv;
          } else {
            ((__bf16*)p.dk)[(int64_t)h * p.kgsh + row * p.kgst + ch] = (__bf16)gk;
            ((__bf16*)p.dv)[(int64_t)h * p.kgsh + row * p.kgst + ch] = (__bf16)gv;
          }
        }
      }
    }
  }
}

// The same with the query-side tiles loaded synchronously per query tile:
// for query tiles larger than key tiles, whose two-stage rings would leave
// one wave per SIMD (LDS).
template <int QT, int KT, bool LM>
__global__ __launch_bounds__(KT * 2) void bwd_dkdv_sync_kernel(BwdParams p) {
  constexpr int W = KT / 32;
  constexpr int NT = W * kWave;
  constexpr int QC = QT / 32;  // 32-query chunks per query tile
  __shared__ u32x4 qs_t[QT * 8], ds_t[QT * 8];  // Q and dout tiles (QT rows x 128 B)
  __shared__ float lse_s[QT], dsum_s[QT];
  const lds_u8* qtile = (const lds_u8*)qs_t;
  const lds_u8* dtile = (const lds_u8*)ds_t;
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int hh = lane >> 5, kl = lane & 31;
  const int n_blocks = LM ? (p.tk + KT - 1) / KT : p.tk;
  const bool gf = p.g_f32 != 0;
  const int h = blockIdx.y;
  for (int cb = blockIdx.x; cb < n_blocks; cb += gridDim.x) {
    // this lane's column (key token or landmark row) and its validity
    const int col = KT * cb + 32 * wave + kl;
    int rows_valid;  // valid columns of the block
    const uint16_t* kb;
    const uint16_t* vb;
    int64_t kstride;
    if constexpr (LM) {
      rows_valid = min(KT, p.tk - KT * cb);
      kb = p.kbar_b + (int64_t)h * p.tk * kHeadDim;
      vb = p.vbar_b + (int64_t)h * p.tk * kHeadDim;
      kstride = kHeadDim;
    } else {
      rows_valid = (int)min<int64_t>(KT, p.nk - (int64_t)KT * cb);
      kb = p.k + (int64_t)h * p.ksh;
      vb = p.v + (int64_t)h * p.ksh;
      kstride = p.kst;
    }
    const int lcol = 32 * wave + kl;  // column within the block
    const bool cvalid = lcol < rows_valid;
    // B operands K^T and V^T of this lane's column: channels 16 s + 8 hh .. +7
    bf16x8 kop[4], vop[4];
    {
      const int64_t row = (int64_t)KT * cb + (cvalid ? lcol : 0);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
        if (cvalid) {
          a = *(const u32x4*)(kb + row * kstride + 16 * s + 8 * hh);
          b = *(const u32x4*)(vb + row * kstride + 16 * s + 8 * hh);
        }
        kop[s] = as_bf16x8(a);
        vop[s] = as_bf16x8(b);
      }
    }
    // logit bias of the column in log2 units (landmarks under the log count)
    float bias = 0.f;
    if constexpr (LM) {
      if (p.log_count) {
        bias = p.lm_log2_kt;
        const int64_t tail = p.nk - (int64_t)(p.tk - 1) * KT;
        if (col == p.tk - 1 && tail < KT) bias += p.lm_tail_corr * p.c;
      }
    }
    f32x16 dkacc[2], dvacc[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      dkacc[0][i] = 0.f;
      dkacc[1][i] = 0.f;
      dvacc[0][i] = 0.f;
      dvacc[1][i] = 0.f;
    }
    int n_i, i_base;
    if constexpr (LM) {
      n_i = p.q_hi - p.q_lo;
      i_base = p.q_lo;
    } else {  // the part of the (ascending) list inside [q_lo, q_hi)
      const int32_t* oh = p.list_off + (int64_t)h * (p.tk + 1);
      const int b0 = oh[cb], b1 = oh[cb + 1];
      i_base = lower_bound_i32(p.list, b0, b1, p.q_lo);
      n_i = lower_bound_i32(p.list, i_base, b1, p.q_hi) - i_base;
    }
    if (n_i == 0 && !p.first && !p.last) continue;  // nothing to add in this launch
    for (int ii = 0; ii < n_i; ++ii) {
      // (a selection with repeated entries would leave list slots unwritten)
      const int qt = LM ? i_base + ii : min(max(p.list[i_base + ii], 0), p.tq - 1);
      // kept mask of this lane's landmark column for query tile qt
      bool masked = !cvalid;
      if constexpr (LM) {
        const int wi = (KT * cb + 32 * wave) / 32;  // the word of this wave's 32 columns
        const uint32_t word =
            wi < p.bit_words ? p.bits[((int64_t)h * p.tq + qt) * p.bit_words + wi] : 0u;
        masked = masked || ((word >> kl) & 1u);
      }
      __syncthreads();  // previous tiles consumed
      for (int e = tid; e < QT * 8; e += NT) {
        const int r = e >> 3, c8 = e & 7;
        const int64_t qrow = (int64_t)qt * QT + r;
        u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
        if (qrow < p.nq) {
          a = *(const u32x4*)(p.q + (int64_t)h * p.qsh + qrow * p.qst + 8 * c8);
          b = load8_bf16(p.dout, (int64_t)h * p.dsh + qrow * p.dst + 8 * c8, gf);
        }
        *(__attribute__((address_space(3))) u32x4*)(qtile + swz(r, c8)) = a;
        *(__attribute__((address_space(3))) u32x4*)(dtile + swz(r, c8)) = b;
      }
      for (int r = tid; r < QT; r += NT) {
        const int64_t qrow = (int64_t)qt * QT + r;
        const bool ok = qrow < p.nq;
        lse_s[r] = ok ? p.lse[(int64_t)h * p.nq + qrow] : INFINITY;
        dsum_s[r] = ok ? p.dsum[(int64_t)h * p.nq + qrow] : 0.f;
      }
      __syncthreads();
#pragma unroll
      for (int qc = 0; qc < QC; ++qc) {
        // S = Q K^T and dP = dout V^T for 32 queries x this wave's 32 columns:
        // lane = column, register v = query 32 qc + 8 (v / 4) + 4 hh + v % 4
        f32x16 sacc, pacc;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const bf16x8 aq = row_operand(qtile, 32 * qc + kl, s, hh);
          const bf16x8 ad = row_operand(dtile, 32 * qc + kl, s, hh);
          if (s == 0) {
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, kop[0], f32x16{}, 0, 0, 0);
            pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ad, vop[0], f32x16{}, 0, 0, 0);
          } else {
            sacc = mfma32(aq, kop[s], sacc);
            pacc = mfma32(ad, vop[s], pacc);
          }
        }
        float pr[16], dsr[16];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int q0 = 32 * qc + 8 * g + 4 * hh;
          const f32x4 l4 = *(const __attribute__((address_space(3))) f32x4*)&lse_s[q0];
          const f32x4 d4 = *(const __attribute__((address_space(3))) f32x4*)&dsum_s[q0];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = 4 * g + r;
            const float pv = masked ? 0.f
                                    : __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[i], p.c, bias) -
                                                             l4[r]);
            pr[i] = pv;
            dsr[i] = pv * (pacc[i] - d4[r]);
          }
        }
        bf16x8 plo, phi, slo, shi, slo2, shi2;
        pack16(pr, plo, phi);
        pack16_split(dsr, slo, shi, slo2, shi2);
        // dV += P^T dout, dK += dS^T Q over these 32 queries (two 16-query chunks)
#pragma unroll
        for (int db = 0; db < 2; ++db) {
          const bf16x8 d0 = tr_operand(dtile, 2 * qc, db, lane);
          const bf16x8 d1 = tr_operand(dtile, 2 * qc + 1, db, lane);
          const bf16x8 q0 = tr_operand(qtile, 2 * qc, db, lane);
          const bf16x8 q1 = tr_operand(qtile, 2 * qc + 1, db, lane);
          dvacc[db] = mfma32(plo, d0, dvacc[db]);
          dvacc[db] = mfma32(phi, d1, dvacc[db]);
          dkacc[db] = mfma32(slo, q0, dkacc[db]);
          dkacc[db] = mfma32(shi, q1, dkacc[db]);
          dkacc[db] = mfma32(slo2, q0, dkacc[db]);
          dkacc[db] = mfma32(shi2, q1, dkacc[db]);
        }
      }
    }
    // epilogue: lane holds channel 32 db + kl of rows (columns of the block)
    // 32 wave + 8 (v / 4) + 4 hh + v % 4
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      const int ch = 32 * db + kl;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int lc = 32 * wave + 8 * (v >> 2) + 4 * hh + (v & 3);
        if (lc >= rows_valid) continue;
        const int64_t row = (int64_t)KT * cb + lc;
        float gk = p.scale * dkacc[db][v];
        float gv = dvacc[db][v];
        float* ak = LM ? p.dkbar : p.acc_k;
        float* av = LM ? p.dvbar : p.acc_v;
        const int64_t ai = ((int64_t)h * (LM ? p.tk : p.nk) + row) * kHeadDim + ch;
        if (!p.first) {  // add this launch's query tiles to the earlier ones
          gk += ak[ai];
          gv += av[ai];
        }
        if (LM || !p.last) {
          ak[ai] = gk;
          av[ai] = gv;
        } else {
          if (p.landmarks && p.dkbar != nullptr) {  // this tile's landmark share
            const float inv_n = 1.0f / (float)rows_valid;
            gk += p.dkbar[((int64_t)h * p.tk + cb) * kHeadDim + ch] * inv_n;
            gv += p.dvbar[((int64_t)h * p.tk + cb) * kHeadDim + ch] * inv_n;
          }
          if (gf) {
            ((float*)p.dk)[(int64_t)h * p.kgsh + row * p.kgst + ch] = gk;
            ((float*)p.dv)[(int64_t)h * p.kgsh + row * p.kgst + ch] = gv;
          } else {
            ((__bf16*)p.dk)[(int64_t)h * p.kgsh + row * p.kgst + ch] = (__bf16)gk;
            ((__bf16*)p.dv)[(int64_t)h * p.kgsh + row * p.kgst + ch] = (__bf16)gv;
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 5. dq: one workgroup per (head, query tile); wave w owns 32 queries
// ---------------------------------------------------------------------------
template <int QT, int KT, bool kGrad>
__global__ __launch_bounds__(QT * 2) __attribute__((amdgpu_waves_per_eu(2))) void bwd_dq_kernel(BwdParams p) {
  constexpr int W = QT / 32;
  constexpr int NB = KT / 32;
  constexpr int KB = KT * 128 / 1024;  // 1 KB pieces per K (or V) block
  constexpr int NU = KB / W;           // pieces per wave per tensor
  static_assert(KB % W == 0, "load split");
  // Two-stage rings, loaded global -> LDS directly one block ahead. Distinct
  // arrays indexed with compile-time stage numbers let the compiler tell the
  // stage being read from the stage being loaded.
  __shared__ u32x4 ks0[KT * 8], vs0[KT * 8], ks1[KT * 8], vs1[KT * 8];
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int qi = lane & 31, hh = lane >> 5;
  const bool gf = p.g_f32 != 0;
  const int n_lb_all = p.landmarks ? (p.tk + KT - 1) / KT : 0;
  const int tail_rows = (int)(p.nk - (int64_t)(p.tk - 1) * KT);
  const int last_lrows = p.tk - (n_lb_all - 1) * KT;
  // piece v of a block: rows 8 (wave + W v) + lane / 8; the lane writes
  // physical chunk lane % 8, i.e. logical chunk (lane % 8) ^ swz_f(row) of
  // the row (the swizzled layout the operand reads expect)
  const int lrow = lane >> 3;
  // byte offsets of the lane's 16 bytes of piece v within a staged block: key
  // rows p.kst elements apart, landmark rows 64
  uint32_t off_kv[NU], off_lm[NU];
#pragma unroll
  for (int v = 0; v < NU; ++v) {
    const int r = 8 * (wave + W * v) + lrow;
    const uint32_t c16 = 16u * (uint32_t)((lane & 7) ^ swz_f(r));
    off_kv[v] = (uint32_t)r * (uint32_t)p.kst * 2u + c16;
    off_lm[v] = (uint32_t)r * (uint32_t)kHeadDim * 2u + c16;
  }
  // per-lane byte offsets of the operand reads within a staged block (the
  // swizzle depends on row bits 1-3 only, so 16- and 32-row steps are plain
  // offsets): row operands of key row qi, chunk 2 s + hh; transposed
  // operands at rows r0 and r0 + 8 of the lane's channel block db
  uint32_t koff[4], toff[2][2];
#pragma unroll
  for (int s = 0; s < 4; ++s) koff[s] = swz(qi, 2 * s + hh);
  {
    const int G = lane >> 4, S = lane & 15;
    const int r0 = 4 * (G >> 1) + (S >> 2);
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      const int col = 32 * db + 16 * (G & 1) + 4 * (S & 3);
      const int chunk = col >> 3, half = (col & 7) ? 8 : 0;
      toff[db][0] = swz(r0, chunk) + half;
      toff[db][1] = swz(r0 + 8, chunk) + half;
    }
  }
  auto row_op = [&](const lds_u8* tile, int b, int s) -> bf16x8 {
    return as_bf16x8(*(const __attribute__((address_space(3))) u32x4*)(tile + koff[s] + 4096 * b));
  };
  auto tr_op = [&](const lds_u8* tile, int m, int db) -> bf16x8 {
    const i16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(tile + toff[db][0] + 2048 * m));
    const i16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(tile + toff[db][1] + 2048 * m));
    const u32x2 w0 = __builtin_bit_cast(u32x2, t0), w1 = __builtin_bit_cast(u32x2, t1);
    return as_bf16x8(u32x4{w0.x, w0.y, w1.x, w1.y});
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  for (int64_t item = blockIdx.x; item < (int64_t)p.heads * p.tq; item += gridDim.x) {
    const int h = (int)(item / p.tq);
    const int qt = (int)(item - (int64_t)h * p.tq);
    const int64_t row = (int64_t)h * p.tq + qt;
    const int32_t* sel_row = p.sel + row * p.top_k;
    const int64_t qrow = (int64_t)qt * QT + wave * 32 + qi;
    const bool qvalid = qrow < p.nq;
    bf16x8 qop[4], dop[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
      if (qvalid) {
        a = *(const u32x4*)(p.q + (int64_t)h * p.qsh + qrow * p.qst + 16 * s + 8 * hh);
        b = load8_bf16(p.dout, (int64_t)h * p.dsh + qrow * p.dst + 16 * s + 8 * hh, gf);
      }
      qop[s] = as_bf16x8(a);
      dop[s] = as_bf16x8(b);
    }
    const float lse = qvalid ? p.lse[(int64_t)h * p.nq + qrow] : INFINITY;
    // sweep 1: D = sum_c P_c dP_c from sweep 0
    const float dsum = kGrad && qvalid ? p.dsum[(int64_t)h * p.nq + qrow] : 0.f;
    f32x16 dqacc[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      dqacc[0][i] = 0.f;
      dqacc[1][i] = 0.f;
    }
    // this launch's key tiles [k_lo, k_hi): kept entries [t0, t1) of the
    // ascending row, landmark blocks [lb0, lb1)
    const int t0 = lower_bound_i32(sel_row, 0, p.top_k, p.k_lo);
    const int t1 = lower_bound_i32(sel_row, t0, p.top_k, p.k_hi);
    const int lb0 = p.k_lo / KT, lb1 = min(n_lb_all, (p.k_hi + KT - 1) / KT);
    const int n_kept = t1 - t0;
    const int n_total = n_kept + max(lb1 - lb0, 0);
    const uint32_t* brow = p.bits + row * p.bit_words;
    int rot = 0;  // phased walk of the kept tiles
    if (p.phase_period > 0 && n_kept > 1) {
      const int target =
          p.k_lo + (int)((item % p.phase_period) * (p.k_hi - p.k_lo) / p.phase_period);
      const int r = lower_bound_i32(sel_row, t0, t1, target) - t0;
      rot = r < n_kept ? r : 0;
    }
    // block t of the list: kept key tile (ascending) or landmark block
    struct Blk {
      const uint16_t* kbase;
      const uint16_t* vbase;
      int64_t stride;
      int rows;
      bool lm;
      int b;  // landmark block index
    };
    auto blk = [&](int t) -> Blk {
      Blk r;
      r.lm = t >= n_kept;
      if (!r.lm) {
        const int tt = t + rot < n_kept ? t + rot : t + rot - n_kept;
        const int j = min(max(sel_row[t0 + tt], 0), p.tk - 1);
        r.kbase = p.k + (int64_t)h * p.ksh + (int64_t)j * KT * p.kst;
        r.vbase = p.v + (int64_t)h * p.ksh + (int64_t)j * KT * p.kst;
        r.stride = p.kst;
        r.rows = j == p.tk - 1 ? tail_rows : KT;
        r.b = 0;
      } else {
        r.b = lb0 + t - n_kept;
        r.kbase = p.kbar_b + ((int64_t)h * p.tk + (int64_t)r.b * KT) * kHeadDim;
        r.vbase = p.vbar_b + ((int64_t)h * p.tk + (int64_t)r.b * KT) * kHeadDim;
        r.stride = kHeadDim;
        r.rows = r.b == n_lb_all - 1 ? last_lrows : KT;
      }
      return r;
    };
    // stage block t through buffer resources whose records end at the block's
    // last valid row (rows past a short tile read as zeros; they are masked)
    auto issue = [&](int t, auto stc) {
      const Blk bk = blk(t);
      u32x4* kd = decltype(stc)::value == 0 ? ks0 : ks1;
      u32x4* vd = decltype(stc)::value == 0 ? vs0 : vs1;
      const uint32_t bytes = (uint32_t)(((int64_t)(bk.rows - 1) * bk.stride + kHeadDim) * 2);
      const __amdgpu_buffer_rsrc_t rk = rows_rsrc(bk.kbase, bytes);
      const __amdgpu_buffer_rsrc_t rv = rows_rsrc(bk.vbase, bytes);
#pragma unroll
      for (int v = 0; v < NU; ++v) {
        const int u = wave + W * v;
        const uint32_t off = bk.lm ? off_lm[v] : off_kv[v];
        b2l16(rk, &kd[64 * u], off);
        b2l16(rv, &vd[64 * u], off);
      }
    };
    // sweep 0: sum_c P'_c and sum_c P'_c dP_c with P' = 2^(x - lse) in
    // float32. The forward's normaliser sums bf16-rounded probabilities, so P'
    // sums to 1 + O(2^-9); renormalising lse by that sum makes P sum to one in
    // float32, and D = sum P dP then matches dP exactly (dP - D cancels, which
    // would amplify any mismatch). sweep 1: dS and dq.
    float dpart = 0.f, lpart = 0.f;
    // sweep 0: the probabilities of key half 1 of the last fast block, done
    // beside the next block's first MFMAs (or before any other block)
    f32x16 pend_s, pend_p;
    float pend_nb = 0.f;
    bool pending = false;
    auto pend_job = [&](int j) {
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(pend_s[2 * j], p.c, pend_nb));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(pend_s[2 * j + 1], p.c, pend_nb));
      dpart = __builtin_fmaf(p0, pend_p[2 * j], dpart);
      lpart += p0;
      dpart = __builtin_fmaf(p1, pend_p[2 * j + 1], dpart);
      lpart += p1;
    };
    auto flush = [&]() {
      if constexpr (!kGrad) {
        if (pending) {
#pragma unroll
          for (int j = 0; j < 8; ++j) pend_job(j);
          pending = false;
        }
      }
    };
    // A 64-key block without excluded columns, in a fixed instruction order
    // (scheduling fences between MFMA slots) so that each wave's VALU work
    // runs beside its own MFMAs: slots 1-8 S and dP of key half 0 (operand
    // reads of half 1 beside them), slots 9-16 S and dP of half 1 beside the
    // probabilities of half 0 (sweep 1: their dS split into bf16 pairs, and
    // the K^T operand reads of half 0), slots 17-24 dq of half 0 beside the
    // probabilities of half 1, slots 25-32 dq of half 1. Per accumulator the
    // summation order is that of the plain block loop below.
    auto fast_block = [&](auto pend_c, const lds_u8* ktile, const lds_u8* vtile, float nb) {
      constexpr bool pend_here = decltype(pend_c)::value;  // (sweep 0 only)
      bf16x8 ka0[4], va0[4], ka1[4], va1[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        ka0[s] = row_op(ktile, 0, s);
        va0[s] = row_op(vtile, 0, s);
      }
      f32x16 sa0, pa0, sa1, pa1;
      // sweep 0: a pending half of the previous block goes beside slots 1-8
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int s = 0; s < 4; ++s) {  // slots 1-8
        sa0 = s == 0 ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka0[0], qop[0], f32x16{}, 0, 0, 0)
                     : mfma32(ka0[s], qop[s], sa0);
        ka1[s] = row_op(ktile, 1, s);
        if constexpr (pend_here) pend_job(2 * s);
        __builtin_amdgcn_sched_barrier(0);
        pa0 = s == 0 ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(va0[0], dop[0], f32x16{}, 0, 0, 0)
                     : mfma32(va0[s], dop[s], pa0);
        va1[s] = row_op(vtile, 1, s);
        if constexpr (pend_here) pend_job(2 * s + 1);
        __builtin_amdgcn_sched_barrier(0);
      }
      // probabilities (and, in sweep 1, the split dS) of keys 2 j, 2 j + 1
      uint32_t w[8], r[8];
      auto job = [&](const f32x16& sa, const f32x16& pa, int j) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[2 * j], p.c, nb));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[2 * j + 1], p.c, nb));
        if constexpr (kGrad) {
          const float d0 = p0 * (pa[2 * j] - dsum), d1 = p1 * (pa[2 * j + 1] - dsum);
          w[j] = pack_bf16x2(d0, d1);
          r[j] = pack_bf16x2(d0 - bf16lo(w[j]), d1 - bf16hi(w[j]));
        } else {
          dpart = __builtin_fmaf(p0, pa[2 * j], dpart);
          lpart += p0;
          dpart = __builtin_fmaf(p1, pa[2 * j + 1], dpart);
          lpart += p1;
        }
      };
      bf16x8 kt[2][2];  // K^T operands [16-key chunk][channel block]
      auto dq_slot = [&](int j) {  // dq^T += K^T dS^T: (lo, hi, small lo, small hi) per block
        const int db = j & 1, part = j >> 1;
        const int m = part & 1;
        const bf16x8 op = part == 0   ? as_bf16x8(u32x4{w[0], w[1], w[2], w[3]})
                          : part == 1 ? as_bf16x8(u32x4{w[4], w[5], w[6], w[7]})
                          : part == 2 ? as_bf16x8(u32x4{r[0], r[1], r[2], r[3]})
                                      : as_bf16x8(u32x4{r[4], r[5], r[6], r[7]});
        dqacc[db] = mfma32(kt[m][db], op, dqacc[db]);
      };
#pragma unroll
      for (int j = 0; j < 8; ++j) {  // slots 9-16
        const int s = j >> 1;
        if ((j & 1) == 0)
          sa1 = s == 0 ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka1[0], qop[0], f32x16{}, 0, 0, 0)
                       : mfma32(ka1[s], qop[s], sa1);
        else
          pa1 = s == 0 ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(va1[0], dop[0], f32x16{}, 0, 0, 0)
                       : mfma32(va1[s], dop[s], pa1);
        job(sa0, pa0, j);
        if constexpr (kGrad) {
          if (j < 4) kt[j >> 1][j & 1] = tr_op(ktile, j >> 1, j & 1);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (kGrad) {
        // w, r of half 0 are complete; half 1's reuse them after its dq slots
        uint32_t w0[8], r0[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          w0[j] = w[j];
          r0[j] = r[j];
        }
        bf16x8 kt1[2][2];
#pragma unroll
        for (int j = 0; j < 8; ++j) {  // slots 17-24
          const int db = j & 1, part = j >> 1, m = part & 1;
          const bf16x8 op = part == 0   ? as_bf16x8(u32x4{w0[0], w0[1], w0[2], w0[3]})
                            : part == 1 ? as_bf16x8(u32x4{w0[4], w0[5], w0[6], w0[7]})
                            : part == 2 ? as_bf16x8(u32x4{r0[0], r0[1], r0[2], r0[3]})
                                        : as_bf16x8(u32x4{r0[4], r0[5], r0[6], r0[7]});
          dqacc[db] = mfma32(kt[m][db], op, dqacc[db]);
          job(sa1, pa1, j);
          if (j < 4) kt1[j >> 1][j & 1] = tr_op(ktile, 2 + (j >> 1), j & 1);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) kt[j >> 2][(j >> 1) & 1] = kt1[j >> 2][(j >> 1) & 1];
#pragma unroll
        for (int j = 0; j < 8; ++j) {  // slots 25-32
          dq_slot(j);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {  // half 1's probabilities wait for the next block's first slots
        pend_s = sa1;
        pend_p = pa1;
        pend_nb = nb;
        pending = true;
      }
    };
    auto step = [&](int t, auto stc) {
      __syncthreads();  // block t has landed for every wave; the other stage is free
      if (t + 1 < n_total) {
        if constexpr (decltype(stc)::value == 0)
          issue(t + 1, S1{});
        else
          issue(t + 1, S0{});
      }
      const lds_u8* ktile = (const lds_u8*)(decltype(stc)::value == 0 ? ks0 : ks1);
      const lds_u8* vtile = (const lds_u8*)(decltype(stc)::value == 0 ? vs0 : vs1);
      const Blk bk = blk(t);
      uint64_t cmask = 0ull;  // excluded columns (bit set)
      float bias = 0.f;       // log2 units
      int tail_col = -1;
      if (bk.lm) {
        const uint32_t lo = brow[NB * bk.b];
        const uint32_t hi = KT == 64 && 2 * bk.b + 1 < p.bit_words ? brow[2 * bk.b + 1] : 0u;
        cmask = ((uint64_t)hi << 32) | lo;
        if (p.log_count) {
          bias = p.lm_log2_kt;
          if (bk.b == n_lb_all - 1 && tail_rows < KT) tail_col = last_lrows - 1;
        }
      }
      if (bk.rows < KT) cmask |= ~0ull << bk.rows;
      if constexpr (NB == 2) {
        if (cmask == 0ull && tail_col < 0) {
          if (!kGrad && pending)
            fast_block(std::true_type{}, ktile, vtile, bias - lse);
          else
            fast_block(std::false_type{}, ktile, vtile, bias - lse);
          return;
        }
      }
      flush();
      // S^T = K Q^T, dP^T = V dout^T: lane = query, register = key
      // 32 b + 8 (v / 4) + 4 hh + v % 4
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        f32x16 sacc, pacc;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const bf16x8 ak = row_op(ktile, b, s);
          const bf16x8 av = row_op(vtile, b, s);
          if (s == 0) {
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, qop[0], f32x16{}, 0, 0, 0);
            pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, dop[0], f32x16{}, 0, 0, 0);
          } else {
            sacc = mfma32(ak, qop[s], sacc);
            pacc = mfma32(av, dop[s], pacc);
          }
        }
        // excluded columns (landmark blocks, a short last tile) as -inf
        // scores and the short last landmark's correction, with uniform lane
        // masks (register v holds key 32 b + 8 (v / 4) + 4 hh + v % 4); the
        // other blocks skip both
        if (cmask != 0ull || tail_col >= 0) {
          const uint32_t w = (uint32_t)(cmask >> (32 * b));
          const uint32_t tw =
              tail_col >= 32 * b && tail_col < 32 * b + 32 ? 1u << (tail_col - 32 * b) : 0u;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int off = 8 * (v >> 2) + (v & 3);
            if (__builtin_amdgcn_inverse_ballot_w64(half_lanes(tw, off)))
              sacc[v] += p.lm_tail_corr;
            if (__builtin_amdgcn_inverse_ballot_w64(half_lanes(w, off))) sacc[v] = -INFINITY;
          }
        }
        const float nb = bias - lse;
        float dsr[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[v], p.c, nb));
          if constexpr (kGrad) {
            dsr[v] = pv * (pacc[v] - dsum);
          } else {
            dpart = __builtin_fmaf(pv, pacc[v], dpart);
            lpart += pv;
          }
        }
        if constexpr (kGrad) {
          bf16x8 slo, shi, slo2, shi2;
          pack16_split(dsr, slo, shi, slo2, shi2);
          // dq^T += K^T dS^T over 16-key chunks 2b and 2b + 1
#pragma unroll
          for (int db = 0; db < 2; ++db) {
            const bf16x8 k0 = tr_op(ktile, 2 * b, db);
            const bf16x8 k1 = tr_op(ktile, 2 * b + 1, db);
            dqacc[db] = mfma32(k0, slo, dqacc[db]);
            dqacc[db] = mfma32(k1, shi, dqacc[db]);
            dqacc[db] = mfma32(k0, slo2, dqacc[db]);
            dqacc[db] = mfma32(k1, shi2, dqacc[db]);
          }
        }
      }
    };
    __syncthreads();  // every wave is done with the previous item's rings
    if (n_total > 0) issue(0, S0{});
    int t = 0;
    for (; t + 2 <= n_total; t += 2) {
      step(t, S0{});
      step(t + 1, S1{});
    }
    if (t < n_total) step(t, S0{});
    flush();
    if constexpr (!kGrad) {  // add this launch's sums over both lane halves
      const auto sd = __builtin_amdgcn_permlane32_swap(__float_as_uint(dpart),
                                                       __float_as_uint(dpart), false, false);
      const auto sl = __builtin_amdgcn_permlane32_swap(__float_as_uint(lpart),
                                                       __float_as_uint(lpart), false, false);
      float dtot = __uint_as_float(sd[0]) + __uint_as_float(sd[1]);
      float ltot = __uint_as_float(sl[0]) + __uint_as_float(sl[1]);
      if (qvalid && hh == 0) {
        const int64_t qi2 = (int64_t)h * p.nq + qrow;
        if (!p.first) {
          dtot += p.d_acc[qi2];
          ltot += p.l_acc[qi2];
        }
        p.d_acc[qi2] = dtot;
        p.l_acc[qi2] = ltot;
      }
    } else if (qvalid) {
      // epilogue: lane (qi, hh) holds channels 32 db + 8 g + 4 hh + r
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t ai = ((int64_t)h * p.nq + qrow) * kHeadDim + 32 * db + 8 * g + 4 * hh;
          f32x4 x = {dqacc[db][4 * g], dqacc[db][4 * g + 1], dqacc[db][4 * g + 2],
                     dqacc[db][4 * g + 3]};
          if (!p.first) x += *(const f32x4*)(p.dq_acc + ai);
          if (!p.last) {
            *(f32x4*)(p.dq_acc + ai) = x;
            continue;
          }
          x *= p.scale;
          const int64_t base = (int64_t)h * p.qgsh + qrow * p.qgst + 32 * db + 8 * g + 4 * hh;
          if (gf)
            *(f32x4*)((float*)p.dq + base) = x;
          else
            *(u32x2*)((uint16_t*)p.dq + base) = u32x2{pack_bf16x2(x[0], x[1]),
                                                      pack_bf16x2(x[2], x[3])};
        }
    }
  }
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0f70 | (N & 15) | ((N >> 4) << 14));
}

// dq for 64-query and 64-key tiles in the key-half layout (kGrad: sweep 1,
// dS and dq; otherwise sweep 0, the sums of P' and P' dP): wave kh
// takes all 64 queries of the tile over keys 32 kh .. 32 kh + 31 of every
// block (S^T = K Q^T, dP^T = V dout^T, dq^T += K^T dS^T), so each K or V
// operand read from LDS feeds both query halves. A wave stages only its own
// rows of a block, global -> LDS directly, into two-stage rings: at the end
// of step t, once its reads of the stage have completed, it refills that
// stage with block t + 2, and step t + 1 waits only for the wave's own loads
// of block t + 1. The steps need no workgroup barrier. The two key halves'
// dq (or sums) meet in LDS at the end of the item, where wave kh keeps query
// half kh. Per block and wave the products and their summation order are
// those of bwd_dq_kernel's half kh of the block.
template <bool kGrad>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2))) void bwd_dq_kh_kernel(
    BwdParams p) {
  constexpr int KT = 64, QT = 64;
  __shared__ u32x4 ks0[KT * 8], vs0[KT * 8], ks1[KT * 8], vs1[KT * 8];
  const int tid = threadIdx.x, lane = tid % kWave;
  const int kh = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int qi = lane & 31, hh = lane >> 5;
  const bool gf = p.g_f32 != 0;
  const int n_lb_all = p.landmarks ? (p.tk + KT - 1) / KT : 0;
  const int tail_rows = (int)(p.nk - (int64_t)(p.tk - 1) * KT);
  const int last_lrows = p.tk - (n_lb_all - 1) * KT;
  // this wave's pieces 4 kh + v (v = 0..3) of a block: rows 8 (4 kh + v) +
  // lane / 8, logical chunk (lane % 8) ^ swz_f(row) landing at physical chunk
  // lane % 8 (the swizzled layout the operand reads expect)
  const int lrow = lane >> 3;
  uint32_t off_kv[4], off_lm[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int r = 8 * (4 * kh + v) + lrow;
    const uint32_t c16 = 16u * (uint32_t)((lane & 7) ^ swz_f(r));
    off_kv[v] = (uint32_t)r * (uint32_t)p.kst * 2u + c16;
    off_lm[v] = (uint32_t)r * (uint32_t)kHeadDim * 2u + c16;
  }
  // operand reads: row operands of key row 32 kh + qi, chunk 2 s + hh;
  // transposed operands at rows r0 and r0 + 8 of 16-key chunk m = 2 kh + mm
  uint32_t koff[4], toff[2][2];
#pragma unroll
  for (int s = 0; s < 4; ++s) koff[s] = swz(qi, 2 * s + hh) + 4096u * (uint32_t)kh;
  {
    const int G = lane >> 4, S = lane & 15;
    const int r0 = 4 * (G >> 1) + (S >> 2);
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      const int col = 32 * db + 16 * (G & 1) + 4 * (S & 3);
      const int chunk = col >> 3, half = (col & 7) ? 8 : 0;
      toff[db][0] = swz(r0, chunk) + half + 4096u * (uint32_t)kh;
      toff[db][1] = swz(r0 + 8, chunk) + half + 4096u * (uint32_t)kh;
    }
  }
  auto row_op = [&](const lds_u8* tile, int s) -> bf16x8 {
    return as_bf16x8(*(const __attribute__((address_space(3))) u32x4*)(tile + koff[s]));
  };
  auto tr_op = [&](const lds_u8* tile, int mm, int db) -> bf16x8 {
    const i16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(tile + toff[db][0] + 2048 * mm));
    const i16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(tile + toff[db][1] + 2048 * mm));
    const u32x2 w0 = __builtin_bit_cast(u32x2, t0), w1 = __builtin_bit_cast(u32x2, t1);
    return as_bf16x8(u32x4{w0.x, w0.y, w1.x, w1.y});
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  for (int64_t item = blockIdx.x; item < (int64_t)p.heads * p.tq; item += gridDim.x) {
    const int h = (int)(item / p.tq);
    const int qt = (int)(item - (int64_t)h * p.tq);
    const int64_t row = (int64_t)h * p.tq + qt;
    const int32_t* sel_row = p.sel + row * p.top_k;
    bf16x8 qop[2][4], dop[2][4];
    float lse[2], dsum[2];
#pragma unroll
    for (int qh = 0; qh < 2; ++qh) {
      const int64_t qrow = (int64_t)qt * QT + 32 * qh + qi;
      const bool qvalid = qrow < p.nq;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
        if (qvalid) {
          a = *(const u32x4*)(p.q + (int64_t)h * p.qsh + qrow * p.qst + 16 * s + 8 * hh);
          b = load8_bf16(p.dout, (int64_t)h * p.dsh + qrow * p.dst + 16 * s + 8 * hh, gf);
        }
        qop[qh][s] = as_bf16x8(a);
        dop[qh][s] = as_bf16x8(b);
      }
      lse[qh] = qvalid ? p.lse[(int64_t)h * p.nq + qrow] : INFINITY;
      dsum[qh] = kGrad && qvalid ? p.dsum[(int64_t)h * p.nq + qrow] : 0.f;
    }
    // sweep 0: per query half, sum_c P'_c dP_c and sum_c P'_c over this wave's keys
    float dpart[2] = {0.f, 0.f}, lpart[2] = {0.f, 0.f};
    f32x16 dqacc[2][2];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      dqacc[0][0][i] = 0.f;
      dqacc[0][1][i] = 0.f;
      dqacc[1][0][i] = 0.f;
      dqacc[1][1][i] = 0.f;
    }
    // this launch's key tiles [k_lo, k_hi): kept entries [t0, t1) of the
    // ascending row, landmark blocks [lb0, lb1)
    const int t0 = lower_bound_i32(sel_row, 0, p.top_k, p.k_lo);
    const int t1 = lower_bound_i32(sel_row, t0, p.top_k, p.k_hi);
    const int lb0 = p.k_lo / KT, lb1 = min(n_lb_all, (p.k_hi + KT - 1) / KT);
    const int n_kept = t1 - t0;
    const int n_total = n_kept + max(lb1 - lb0, 0);
    // the kept list and bits as constant memory (scalar loads)
    const cint_p sel_c = (cint_p)sel_row;
    const cuint_p brow = (cuint_p)(p.bits + row * p.bit_words);
    int rot = 0;  // phased walk of the kept tiles
    if (p.phase_period > 0 && n_kept > 1) {
      const int target =
          p.k_lo + (int)((item % p.phase_period) * (p.k_hi - p.k_lo) / p.phase_period);
      const int r = lower_bound_i32(sel_row, t0, t1, target) - t0;
      rot = r < n_kept ? r : 0;
    }
    // block t of the list: kept key tile (walk order) or landmark block
    struct Blk {
      const uint16_t* kbase;
      const uint16_t* vbase;
      int64_t stride;
      int rows;
      bool lm;
      int b;  // landmark block index
    };
    auto blk = [&](int t) -> Blk {
      Blk r;
      r.lm = t >= n_kept;
      if (!r.lm) {
        const int tt = t + rot < n_kept ? t + rot : t + rot - n_kept;
        const int j = min(max(sel_c[t0 + tt], 0), p.tk - 1);
        r.kbase = p.k + (int64_t)h * p.ksh + (int64_t)j * KT * p.kst;
        r.vbase = p.v + (int64_t)h * p.ksh + (int64_t)j * KT * p.kst;
        r.stride = p.kst;
        r.rows = j == p.tk - 1 ? tail_rows : KT;
        r.b = 0;
      } else {
        r.b = lb0 + t - n_kept;
        r.kbase = p.kbar_b + ((int64_t)h * p.tk + (int64_t)r.b * KT) * kHeadDim;
        r.vbase = p.vbar_b + ((int64_t)h * p.tk + (int64_t)r.b * KT) * kHeadDim;
        r.stride = kHeadDim;
        r.rows = r.b == n_lb_all - 1 ? last_lrows : KT;
      }
      return r;
    };
    // this wave's rows of block t, through buffer resources whose records end
    // at the block's last valid row (rows past a short tile read as zeros;
    // their columns are masked)
    auto issue = [&](int t, auto stc) {
      const Blk bk = blk(t);
      u32x4* kd = decltype(stc)::value == 0 ? ks0 : ks1;
      u32x4* vd = decltype(stc)::value == 0 ? vs0 : vs1;
      const uint32_t bytes = (uint32_t)(((int64_t)(bk.rows - 1) * bk.stride + kHeadDim) * 2);
      const __amdgpu_buffer_rsrc_t rk = rows_rsrc(bk.kbase, bytes);
      const __amdgpu_buffer_rsrc_t rv = rows_rsrc(bk.vbase, bytes);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int u = 4 * kh + v;
        const uint32_t off = bk.lm ? off_lm[v] : off_kv[v];
        b2l16(rk, &kd[64 * u], off);
        b2l16(rv, &vd[64 * u], off);
      }
    };
    auto step = [&](int t, auto stc) {
      // this wave's loads of block t have landed; block t + 1's may be in
      // flight (every step issues one block: past the end, the last again)
      wait_vm<8>();
      const lds_u8* ktile = (const lds_u8*)(decltype(stc)::value == 0 ? ks0 : ks1);
      const lds_u8* vtile = (const lds_u8*)(decltype(stc)::value == 0 ? vs0 : vs1);
      const Blk bk = blk(t);
      uint64_t cmask = 0ull;  // excluded columns (bit set)
      float bias = 0.f;       // log2 units
      int tail_col = -1;
      if (bk.lm) {
        const uint32_t lo = brow[2 * bk.b];
        const uint32_t hi = 2 * bk.b + 1 < p.bit_words ? brow[2 * bk.b + 1] : 0u;
        cmask = ((uint64_t)hi << 32) | lo;
        if (p.log_count) {
          bias = p.lm_log2_kt;
          if (bk.b == n_lb_all - 1 && tail_rows < KT) tail_col = last_lrows - 1;
        }
      }
      if (bk.rows < KT) cmask |= ~0ull << bk.rows;
      const uint32_t wm = (uint32_t)(cmask >> (32 * kh));
      const uint32_t tw = tail_col >= 32 * kh && tail_col < 32 * kh + 32
                              ? 1u << (tail_col - 32 * kh) : 0u;
      bf16x8 kr[4], vr[4], kt[2][2];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        kr[s] = row_op(ktile, s);
        vr[s] = row_op(vtile, s);
      }
      if constexpr (kGrad) {
#pragma unroll
        for (int mm = 0; mm < 2; ++mm)
#pragma unroll
          for (int db = 0; db < 2; ++db) kt[mm][db] = tr_op(ktile, mm, db);
      }
#pragma unroll
      for (int qh = 0; qh < 2; ++qh) {
        // S^T = K Q^T, dP^T = V dout^T: lane = query, register v = key
        // 32 kh + 8 (v / 4) + 4 hh + v % 4
        f32x16 sacc, pacc;
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[0], qop[qh][0], f32x16{}, 0, 0, 0);
        pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vr[0], dop[qh][0], f32x16{}, 0, 0, 0);
#pragma unroll
        for (int s = 1; s < 4; ++s) {
          sacc = mfma32(kr[s], qop[qh][s], sacc);
          pacc = mfma32(vr[s], dop[qh][s], pacc);
        }
        if (wm != 0u || tw != 0u) {
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int off = 8 * (v >> 2) + (v & 3);
            if (__builtin_amdgcn_inverse_ballot_w64(half_lanes(tw, off)))
              sacc[v] += p.lm_tail_corr;
            if (__builtin_amdgcn_inverse_ballot_w64(half_lanes(wm, off))) sacc[v] = -INFINITY;
          }
        }
        const float nb = bias - lse[qh];
        if constexpr (!kGrad) {
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[v], p.c, nb));
            dpart[qh] = __builtin_fmaf(pv, pacc[v], dpart[qh]);
            lpart[qh] += pv;
          }
          continue;
        }
        float dsr[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[v], p.c, nb));
          dsr[v] = pv * (pacc[v] - dsum[qh]);
        }
        bf16x8 slo, shi, slo2, shi2;
        pack16_split(dsr, slo, shi, slo2, shi2);
        // dq^T += K^T dS^T over this wave's 16-key chunks
#pragma unroll
        for (int db = 0; db < 2; ++db) {
          dqacc[qh][db] = mfma32(kt[0][db], slo, dqacc[qh][db]);
          dqacc[qh][db] = mfma32(kt[1][db], shi, dqacc[qh][db]);
          dqacc[qh][db] = mfma32(kt[0][db], slo2, dqacc[qh][db]);
          dqacc[qh][db] = mfma32(kt[1][db], shi2, dqacc[qh][db]);
        }
      }
      // refill this stage with block t + 2 once the reads above have
      // completed: an LDS write by a global load is not ordered after LDS
      // reads still in flight
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      issue(min(t + 2, n_total - 1), stc);
    };
    __syncthreads();  // both waves are done with the previous item's LDS
    if (n_total > 0) {
      issue(0, S0{});
      issue(min(1, n_total - 1), S1{});
      int t = 0;
      for (; t + 2 <= n_total; t += 2) {
        step(t, S0{});
        step(t + 1, S1{});
      }
      if (t < n_total) step(t, S0{});
      wait_vm<0>();  // the repeated last blocks have landed
    }
    // the key halves meet: wave kh hands query half 1 - kh to its partner
    // through the idle rings
    __syncthreads();
    if constexpr (!kGrad) {
      // sums over the lane halves (they hold different keys of a query), then
      // over the two key halves; wave kh writes query half kh
      float dq2[2], lq2[2];
#pragma unroll
      for (int qh = 0; qh < 2; ++qh) {
        const auto sd = __builtin_amdgcn_permlane32_swap(__float_as_uint(dpart[qh]),
                                                         __float_as_uint(dpart[qh]), false, false);
        const auto sl = __builtin_amdgcn_permlane32_swap(__float_as_uint(lpart[qh]),
                                                         __float_as_uint(lpart[qh]), false, false);
        dq2[qh] = __uint_as_float(sd[0]) + __uint_as_float(sd[1]);
        lq2[qh] = __uint_as_float(sl[0]) + __uint_as_float(sl[1]);
      }
      float2* xo = (float2*)(kh == 0 ? ks0 : vs0);
      if (hh == 0) xo[qi] = kh == 0 ? float2{dq2[1], lq2[1]} : float2{dq2[0], lq2[0]};
      __syncthreads();
      const float2 o = ((const float2*)(kh == 0 ? vs0 : ks0))[qi];
      float dtot = (kh == 0 ? dq2[0] : dq2[1]) + o.x;
      float ltot = (kh == 0 ? lq2[0] : lq2[1]) + o.y;
      const int64_t qrow = (int64_t)qt * QT + 32 * kh + qi;
      if (qrow < p.nq && hh == 0) {
        const int64_t qi2 = (int64_t)h * p.nq + qrow;
        if (!p.first) {
          dtot += p.d_acc[qi2];
          ltot += p.l_acc[qi2];
        }
        p.d_acc[qi2] = dtot;
        p.l_acc[qi2] = ltot;
      }
      continue;
    }
    // (kh is uniform: both branches index the register arrays statically)
    auto put = [&](const f32x16 (&a)[2], f32x4* xo) {
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          xo[(db * 4 + g) * 64 + lane] =
              f32x4{a[db][4 * g], a[db][4 * g + 1], a[db][4 * g + 2], a[db][4 * g + 3]};
    };
    if (kh == 0)
      put(dqacc[1], (f32x4*)ks0);
    else
      put(dqacc[0], (f32x4*)vs0);
    __syncthreads();
    auto finish = [&](const f32x16 (&a)[2], const f32x4* xi) {
      const int64_t qrow = (int64_t)qt * QT + 32 * kh + qi;
      if (qrow >= p.nq) return;
      // lane (qi, hh) holds channels 32 db + 8 g + 4 hh + r
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          // the two key halves' sums (float addition is commutative, so
          // both waves form the same value)
          f32x4 x = f32x4{a[db][4 * g], a[db][4 * g + 1], a[db][4 * g + 2], a[db][4 * g + 3]} +
                    xi[(db * 4 + g) * 64 + lane];
          const int64_t ai = ((int64_t)h * p.nq + qrow) * kHeadDim + 32 * db + 8 * g + 4 * hh;
          if (!p.first) x += *(const f32x4*)(p.dq_acc + ai);
          if (!p.last) {
            *(f32x4*)(p.dq_acc + ai) = x;
            continue;
          }
          x *= p.scale;
          const int64_t base = (int64_t)h * p.qgsh + qrow * p.qgst + 32 * db + 8 * g + 4 * hh;
          if (gf)
            *(f32x4*)((float*)p.dq + base) = x;
          else
            *(u32x2*)((uint16_t*)p.dq + base) = u32x2{pack_bf16x2(x[0], x[1]),
                                                      pack_bf16x2(x[2], x[3])};
        }
    };
    if (kh == 0)
      finish(dqacc[0], (const f32x4*)vs0);
    else
      finish(dqacc[1], (const f32x4*)ks0);
  }
}

// after the sweep-0 launches: renormalise lse by the sum of P' and form D
__global__ __launch_bounds__(256) void bwd_finalize_kernel(float* __restrict__ lse,
                                                           float* __restrict__ dsum,
                                                           const float* __restrict__ l_acc,
                                                           const float* __restrict__ d_acc,
                                                           int64_t n) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= n) return;
  const float l = l_acc[e];
  lse[e] += __builtin_log2f(l);
  dsum[e] = d_acc[e] / l;
}

size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

struct BwdLayout {
  size_t fwd, dqacc, lse, dsum, lacc, dacc, dkbar, dvbar, acck, accv, doutb, bits, count, off,
      list, total;
};

BwdLayout bwd_layout(int64_t nq, int64_t nk, int32_t heads, int32_t q_tile, int32_t k_tile,
                     int32_t top_k) {
  BwdLayout L;
  const int64_t tq = (nq + q_tile - 1) / q_tile, tk = (nk + k_tile - 1) / k_tile;
  L.fwd = a256(sparse_workspace_bytes(nq, nk, heads, q_tile, k_tile, top_k));
  L.dqacc = a256((size_t)heads * nq * kHeadDim * sizeof(float));  // also the forward's output
  L.lse = a256((size_t)heads * nq * sizeof(float));
  L.dsum = L.lse;
  L.lacc = L.lse;
  L.dacc = L.lse;
  L.dkbar = a256((size_t)heads * tk * kHeadDim * sizeof(float));
  L.dvbar = L.dkbar;
  L.acck = a256((size_t)heads * nk * kHeadDim * sizeof(float));
  L.accv = L.acck;
  L.doutb = a256((size_t)heads * nq * kHeadDim * sizeof(uint16_t));
  L.bits = a256((size_t)heads * tq * ((tk + 31) / 32) * sizeof(uint32_t));
  L.count = a256((size_t)heads * tk * sizeof(int32_t));
  L.off = a256((size_t)heads * (tk + 1) * sizeof(int32_t));
  L.list = a256((size_t)heads * tq * top_k * sizeof(int32_t));
  L.total = L.fwd + L.dqacc + L.lse + L.dsum + L.lacc + L.dacc + L.dkbar + L.dvbar + L.acck +
            L.accv + L.doutb + L.bits + L.count + L.off + L.list;
  return L;
}

// Chunks: the workgroups of one launch share about 8 MB of K and V (dq) or Q
// and dout (dk, dv), which then stay in L2, as in the forward's split keys.
constexpr int kChunkRows = 32768;

// Workgroups of kernel K (with the given block size) the current device runs
// at once, or 0 if the runtime cannot say.
template <auto K, int Threads>
int64_t wgs_at_once() {
  static std::atomic<int> per_cu{-1};
  int nb = per_cu.load(std::memory_order_relaxed);
  if (nb < 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, K, Threads, 0) != hipSuccess) {
      (void)hipGetLastError();
      nb = 0;
    }
    per_cu.store(nb, std::memory_order_relaxed);
  }
  int dev = 0, cus = 0;
  if (nb == 0 || hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return (int64_t)nb * cus;
}

// phase period for a launch of `items` workgroups: only when it runs many
// rounds of them
inline int64_t phase_for(int64_t items, int64_t at_once) {
  return at_once > 0 && items >= 4 * at_once ? at_once : 0;
}

template <int QT, int KT>
hipError_t launch_bwd_kernels(BwdParams p, int32_t heads, bool have_d, hipStream_t s) {
  hipError_t err;
  // dq: sweep 0 over key chunks (sums of P' and P' dP), finalize, sweep 1;
  // with D formed from the forward's float32 output (have_d), sweep 1 alone
  const int ct = kChunkRows / KT;  // key tiles per chunk, a multiple of KT
  const int nkc = (p.tk + ct - 1) / ct;
  const int64_t items = (int64_t)heads * p.tq;
  const dim3 qgrid((unsigned)std::min<int64_t>(items, 1 << 24));
  for (int sweep = have_d ? 1 : 0; sweep < 2; ++sweep) {
    for (int c = 0; c < nkc; ++c) {
      p.k_lo = c * ct;
      p.k_hi = std::min(p.tk, (c + 1) * ct);
      p.first = c == 0;
      p.last = c == nkc - 1;
      if constexpr (QT == 64 && KT == 64) {
        if (sweep == 0) {
          p.phase_period = phase_for(items, wgs_at_once<bwd_dq_kh_kernel<false>, 128>());
          hipLaunchKernelGGL((bwd_dq_kh_kernel<false>), qgrid, dim3(128), 0, s, p);
        } else {
          p.phase_period = phase_for(items, wgs_at_once<bwd_dq_kh_kernel<true>, 128>());
          hipLaunchKernelGGL((bwd_dq_kh_kernel<true>), qgrid, dim3(128), 0, s, p);
        }
      } else if (sweep == 0) {
        p.phase_period = phase_for(items, wgs_at_once<bwd_dq_kernel<QT, KT, false>, QT * 2>());
        hipLaunchKernelGGL((bwd_dq_kernel<QT, KT, false>), qgrid, dim3(QT * 2), 0, s, p);
      } else {
        p.phase_period = phase_for(items, wgs_at_once<bwd_dq_kernel<QT, KT, true>, QT * 2>());
        hipLaunchKernelGGL((bwd_dq_kernel<QT, KT, true>), qgrid, dim3(QT * 2), 0, s, p);
      }
      if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if (sweep == 0) {
      const int64_t n = (int64_t)heads * p.nq;
      hipLaunchKernelGGL(bwd_finalize_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                         p.lse, p.dsum, (const float*)p.l_acc, (const float*)p.d_acc, n);
      if ((err = hipGetLastError()) != hipSuccess) return err;
    }
  }
  // dk, dv: landmark rows, then key tiles, each over query-tile chunks
  const int qch = std::max(1, kChunkRows / QT);
  const int nqc = (p.tq + qch - 1) / qch;
  for (int pass = p.landmarks ? 0 : 1; pass < 2; ++pass) {
    for (int c = 0; c < nqc; ++c) {
      p.q_lo = c * qch;
      p.q_hi = std::min(p.tq, (c + 1) * qch);
      p.first = c == 0;
      p.last = c == nqc - 1;
      const int nb = pass == 0 ? (p.tk + KT - 1) / KT : p.tk;
      const dim3 grid((unsigned)nb, heads);
      // two-stage rings keep two waves per SIMD while QT <= KT (LDS)
      if constexpr (QT <= KT) {
        if (pass == 0) {
          p.phase_period = 0;
          hipLaunchKernelGGL((bwd_dkdv_kernel<QT, KT, true>), grid, dim3(KT * 2), 0, s, p);
        } else {
          p.phase_period = phase_for((int64_t)nb * heads,
                                     wgs_at_once<bwd_dkdv_kernel<QT, KT, false>, KT * 2>());
          hipLaunchKernelGGL((bwd_dkdv_kernel<QT, KT, false>), grid, dim3(KT * 2), 0, s, p);
        }
      } else {
        p.phase_period = 0;
        if (pass == 0)
          hipLaunchKernelGGL((bwd_dkdv_sync_kernel<QT, KT, true>), grid, dim3(KT * 2), 0, s, p);
        else
          hipLaunchKernelGGL((bwd_dkdv_sync_kernel<QT, KT, false>), grid, dim3(KT * 2), 0, s, p);
      }
      if ((err = hipGetLastError()) != hipSuccess) return err;
    }
  }
  return hipSuccess;
}

}  // namespace

size_t sparse_bwd_workspace_bytes(int64_t n_q, int64_t n_kv, int32_t heads, int32_t q_tile,
                                  int32_t k_tile, int32_t top_k) {
  return bwd_layout(n_q, n_kv, heads, q_tile, k_tile, top_k).total;
}

hipError_t launch_tile_sparse_bwd(const uint16_t* q, int64_t nq, int64_t qst, int64_t qsh,
                                  const uint16_t* k, const uint16_t* v, int64_t nk, int64_t kst,
                                  int64_t ksh, int32_t heads, const float* kbar,
                                  const float* vbar, const int32_t* sel, int32_t q_tile,
                                  int32_t k_tile, int32_t top_k, float scale, uint32_t flags,
                                  const void* dout, int64_t dst, int64_t dsh, bool g_f32,
                                  void* dq, int64_t qgst, int64_t qgsh, void* dk, void* dv,
                                  int64_t kgst, int64_t kgsh, void* ws, hipStream_t s,
                                  const float* lse_in, const float* out_in, int64_t ost_in,
                                  int64_t osh_in) {
  if (heads == 0 || (nq == 0 && nk == 0)) return hipSuccess;
  const BwdLayout L = bwd_layout(nq, nk, heads, q_tile, k_tile, top_k);
  uint8_t* w = (uint8_t*)ws;
  uint8_t* cur = w + L.fwd;
  auto take = [&](size_t bytes) {
    uint8_t* r = cur;
    cur += bytes;
    return r;
  };
  float* dq_acc = (float*)take(L.dqacc);
  float* lse = (float*)take(L.lse);
  float* dsum = (float*)take(L.dsum);
  float* l_acc = (float*)take(L.lacc);
  float* d_acc = (float*)take(L.dacc);
  float* dkbar = (float*)take(L.dkbar);
  float* dvbar = (float*)take(L.dvbar);
  float* acc_k = (float*)take(L.acck);
  float* acc_v = (float*)take(L.accv);
  uint16_t* dout_b = (uint16_t*)take(L.doutb);
  uint32_t* bits = (uint32_t*)take(L.bits);
  int32_t* count = (int32_t*)((uint8_t*)bits + L.bits);
  int32_t* off = (int32_t*)((uint8_t*)count + L.count);
  int32_t* list = (int32_t*)((uint8_t*)off + L.off);
  const int32_t tq = (int32_t)((nq + q_tile - 1) / q_tile);
  const int32_t tk = (int32_t)((nk + k_tile - 1) / k_tile);
  const int32_t bit_words = (tk + 31) / 32;
  const bool landmarks = (flags & kSparseNoLandmarks) == 0 && top_k < tk;
  hipError_t err;
  // forward: float32 output and the log2 normaliser (also packs the bf16 landmarks), or,
  // with the normaliser of an earlier forward call given, the landmarks alone and a copy of
  // the normaliser. D = dout . out then comes from the float32 output (the call's own, or
  // the earlier call's when given) and dq needs one sweep; with the normaliser alone the
  // first dq sweep forms D from the probabilities and renormalises the copy in place.
  const bool have_d = lse_in == nullptr || out_in != nullptr;
  const float* o_d = lse_in == nullptr ? dq_acc : out_in;
  const int64_t ost_d = lse_in == nullptr ? kHeadDim : ost_in;
  const int64_t osh_d = lse_in == nullptr ? nq * kHeadDim : osh_in;
  if (nq > 0 && lse_in == nullptr) {
    err = launch_tile_sparse(q, nq, qst, qsh, k, v, nk, kst, ksh, heads, kbar, vbar, sel, q_tile,
                             k_tile, top_k, scale, dq_acc, kHeadDim, nq * kHeadDim, true, flags, w,
                             s, lse);
    if (err != hipSuccess) return err;
  } else if (nq > 0) {
    if (landmarks) {
      const size_t lmb = a256((size_t)heads * tk * kHeadDim * sizeof(uint16_t));
      err = launch_pack_landmarks(kbar, vbar, heads, tk, (uint16_t*)w, (uint16_t*)(w + lmb), s);
      if (err != hipSuccess) return err;
    }
    err = hipMemcpyAsync(lse, lse_in, (size_t)heads * nq * sizeof(float),
                         hipMemcpyDeviceToDevice, s);
    if (err != hipSuccess) return err;
  }
  // dout packed as bf16 rows for the dk, dv kernels' direct-to-LDS staging (and D)
  if (nq > 0) {
    const int64_t pieces = (int64_t)heads * nq * 8;
    hipLaunchKernelGGL(bwd_pack_dout_kernel,
                       dim3((unsigned)std::min<int64_t>((pieces + 255) / 256, 1 << 20)), dim3(256),
                       0, s, dout, dst, dsh, g_f32 ? 1 : 0, nq, pieces, dout_b,
                       have_d ? o_d : nullptr, ost_d, osh_d, dsum);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  // kept bits, counts, offsets, lists
  const int64_t nzero = (int64_t)((uint8_t*)off - (uint8_t*)bits) / 4;  // bits and counts
  hipLaunchKernelGGL(bwd_fill_u32_kernel, dim3((unsigned)std::min<int64_t>((nzero + 255) / 256,
                                                                           4096)),
                     dim3(256), 0, s, bits, nzero);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (tq > 0) {
    const size_t lds = (size_t)(tk + bit_words) * sizeof(uint32_t);
    // the kernel's dynamic LDS limit, raised once per process to what the
    // largest key range (32,768 tiles) needs: 132 KB
    static const hipError_t lds_limit = hipFuncSetAttribute(
        (const void*)bwd_bits_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
        (int)((32768 + 32768 / 32) * sizeof(uint32_t)));
    if (lds_limit != hipSuccess) return lds_limit;
    // about 2,048 workgroups, at most kBitsRows rows each
    const int32_t rpw = (int32_t)std::min<int64_t>(
        kBitsRows, std::max<int64_t>(1, (int64_t)heads * tq / 2048));
    hipLaunchKernelGGL(bwd_bits_kernel, dim3((unsigned)((tq + rpw - 1) / rpw), heads), dim3(256),
                       lds, s, sel, tq, tk, top_k, bit_words, rpw, bits, count);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  hipLaunchKernelGGL(bwd_scan_kernel, dim3(heads), dim3(256), 0, s, count, tk,
                     (int64_t)tq * top_k, off);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(bwd_list_kernel, dim3((unsigned)bit_words, heads), dim3(64), 0, s, bits, tq,
                     tk, bit_words, off, list);
  if ((err = hipGetLastError()) != hipSuccess) return err;

  BwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  // the forward packed the bf16 landmarks at the start of its workspace
  const size_t lm = a256((size_t)heads * tk * kHeadDim * sizeof(uint16_t));
  p.kbar_b = landmarks ? (const uint16_t*)w : nullptr;
  p.vbar_b = landmarks ? (const uint16_t*)(w + lm) : nullptr;
  p.sel = sel;
  p.dout = dout;
  p.dout_b = dout_b;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.nq = nq;
  p.qst = qst;
  p.qsh = qsh;
  p.nk = nk;
  p.kst = kst;
  p.ksh = ksh;
  p.dst = dst;
  p.dsh = dsh;
  p.qgst = qgst;
  p.qgsh = qgsh;
  p.kgst = kgst;
  p.kgsh = kgsh;
  p.heads = heads;
  p.tq = tq;
  p.tk = tk;
  p.top_k = top_k;
  p.bit_words = bit_words;
  p.c = scale * kLog2eB;
  p.scale = scale;
  p.g_f32 = g_f32 ? 1 : 0;
  p.landmarks = landmarks ? 1 : 0;
  p.log_count = (flags & kSparseLandmarkLogCount) ? 1 : 0;
  p.lm_log2_kt = __builtin_log2f((float)k_tile);
  {
    const int64_t tail = nk - (int64_t)(tk - 1) * k_tile;
    p.lm_tail_corr = tail > 0 ? (__builtin_log2f((float)tail) - p.lm_log2_kt) / p.c : 0.f;
  }
  p.lse = lse;
  p.dsum = dsum;
  p.bits = bits;
  p.list_off = off;
  p.list = list;
  p.dkbar = landmarks ? dkbar : nullptr;
  p.dvbar = landmarks ? dvbar : nullptr;
  p.acc_k = acc_k;
  p.acc_v = acc_v;
  p.l_acc = l_acc;
  p.d_acc = d_acc;
  p.dq_acc = dq_acc;
  p.q_lo = p.q_hi = p.k_lo = p.k_hi = p.first = p.last = 0;
  p.phase_period = 0;
  if (k_tile == 64) {
    if (q_tile == 32) return launch_bwd_kernels<32, 64>(p, heads, have_d, s);
    if (q_tile == 64) return launch_bwd_kernels<64, 64>(p, heads, have_d, s);
    return launch_bwd_kernels<128, 64>(p, heads, have_d, s);
  }
  if (q_tile == 32) return launch_bwd_kernels<32, 32>(p, heads, have_d, s);
  if (q_tile == 64) return launch_bwd_kernels<64, 32>(p, heads, have_d, s);
  return launch_bwd_kernels<128, 32>(p, heads, have_d, s);
}

}  // namespace zebra
