// Tile-sparse softmax attention with mean-key/value landmarks (gfx950).
//
// Zebra3D paper page (thelatestinai.com), Figure 1 caption: kept tiles keep
// full softmax interactions; omitted tiles become mean-key/value landmarks.
// For every query of query tile i the softmax runs over every token of the
// kept key tiles sel[h][i][*] plus one landmark column (kbar_j, vbar_j) for
// each omitted tile j. With sel == NULL every tile is kept: exact dense
// attention.
//
// Work decomposition. One workgroup per item, head-major; one wave owns 32
// queries. An item is a list of column blocks of KT columns: its kept key
// tiles (ascending), then the landmark rows of the key tiles it covers, KT at
// a time, with the kept ones masked out by a per-item bitmap in LDS.
// Landmark rows are few and shared by every item of a head, so they stay in
// L2; masking costs less than gathering per-item omitted lists.
//
// Short key ranges (and dense attention): an item is one (head, query tile)
// over every key tile, and writes the normalised output.
//
// Long key ranges (split keys): the key tiles are cut into chunks of CT tiles
// and an item is one (head, key chunk, query tile), ordered chunk-major within
// a head. Query tiles keep different random subsets of key tiles, so over the
// whole range the workgroups running together share almost no K/V blocks and
// every kept block is a fresh fetch from HBM. Within one chunk they share the
// chunk's few megabytes of K/V, which then stay in L2. Each item writes its
// unnormalised output and (reference, row sum) in float32; a combine kernel
// merges the chunks of each query in chunk order:
//   O = sum_c 2^(r_c - R) O_c / sum_c 2^(r_c - R) l_c,   R = max_c r_c.
//
// Per block the wave computes the transposed score block S^T = K Q^T with
// bf16 MFMA 32x32x16 (each lane then holds ONE query's scores over 32 keys),
// the probabilities in float32 rounded to bf16 (already the B-operand layout
// of the second product), and O^T += V^T P^T with V read transposed from LDS
// by ds_read_b64_tr_b16. The row sum is accumulated from the bf16-rounded
// probabilities (v_dot2 with ones), the same values the PV product uses.
//
// Softmax reference. Softmax is invariant to a per-query shift of the
// logits; any shift that keeps exp2 in range gives the same result. The fast
// path uses a bound known before the first block: by Cauchy-Schwarz every
// logit of query q is at most m_q = c |q| max_j |k_j| (c = scale log2 e, max
// over all key and landmark rows of the head, taken by a small prologue
// kernel, with a relative margin for rounding). Probabilities are
// 2^(c s - m_q + 60): at most 2^60, and the largest one is at least
// 2^(60 - 2 m_q) >= 2^-40 when m_q <= 50; with max |v| <= 2^40 and at most
// 2^21 columns nothing overflows or underflows to a significant degree. The
// block loop then has no maximum, no rescale and no branch. Items whose
// bound is too loose take the fallback path: the classic running maximum
// with lazy rescaling (the maximum moves only when a block's maximum exceeds
// it by more than 8 in log2 units).
//
// Variants (the pages' sparse-attention ablations): without landmarks the
// item walks its kept tiles only; with the landmark log count a landmark
// stands for the n_j valid tokens of its tile, i.e. its probability gains a
// factor n_j (2^log2(n_j) in the exponent). The fast path then lowers every
// probability by KT so that the landmarks' stay below 2^60.
//
// Pipeline. K and V blocks go global -> LDS directly
// (global_load_lds_dwordx4) into two-stage rings: step t issues K(t+2) and
// V(t), then computes the softmax of block t (S(t) -> bf16 P(t)) together
// with PV(t-1), and then QK(t+1). The PV product of the previous block does
// not depend on this block's softmax, so each wave's MFMAs run while the
// same wave issues its softmax arithmetic; one score buffer and two P
// buffers (bf16) keep the operands of the next block's reads in registers.
// One barrier per step. 16-byte LDS chunks are XOR swizzled by row so both
// operand reads are bank-conflict free.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "common.h"

namespace zebra {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleSlack = 8.0f;       // fallback path, log2 units
constexpr float kBoundLimit = 50.0f;        // fast path: m_q at most this (log2 units)
constexpr float kPShift = 60.0f;            // fast path: p = 2^(c s - m_q + kPShift)
constexpr float kVLimit = 1099511627776.0f; // fast path: max |v| at most 2^40
constexpr int kWin = 2040;                  // kept-list window entries in LDS
constexpr int kMaxKeyTiles = 32768;
constexpr int kBitWords = kMaxKeyTiles / 32;
constexpr int kRangeParts = 64;             // per-head partial maxima (one per lane)
constexpr int kBufferFlags = 0x00020000;    // buffer resource word 3: 32-bit data format

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;  // LDS bytes

struct SparseParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* kbar_b;  // bf16 landmarks [H][tk][64] (sparse only)
  const uint16_t* vbar_b;
  const float* range;      // [H][kRangeParts][2]: partial max |k|^2, max |v|
  void* o;
  int64_t nq, qst, qsh;
  int64_t nk, kst, ksh;
  int64_t ost, osh;
  int64_t n_items;         // heads * n_chunks * tq
  int32_t tq, tk, top_k;
  float scale_log2;        // softmax scale * log2(e), > 0
  int32_t o_f32;
  int32_t landmarks;       // 0: omitted tiles are dropped (no landmark columns)
  int32_t log_count;       // landmark logits gain log2(n_j) (log2 units)
  float lm_log2_kt;        // log2(KT)
  float lm_tail_corr;      // (log2(n of tile tk-1) - log2(KT)) / c, score units
  // split keys (n_chunks > 1): chunk c covers key tiles [c CT, (c + 1) CT)
  int32_t n_chunks, chunk_tiles;
  const int32_t* coff;     // [H][tq][n_chunks + 1]: first kept entry of each chunk
  float* part_o;           // [H][nq][n_chunks][64] unnormalised outputs
  float2* part_ml;         // [H][nq][n_chunks] (reference, row sum), p = 2^(c s - reference)
  float* lse;              // [H][nq] log2 of the softmax normaliser (log2 units), or null
  // kept-list walk phase (key-half kernel): 0, or the number of items the
  // device runs at once (see the kernel)
  int64_t phase_period;
  // split keys: partial slots per query (n_chunks, plus one for the landmark
  // columns when a separate landmark pass computes them: lm_separate, and the
  // key-chunk items then skip their landmark blocks)
  int32_t part_slots, lm_separate;
  int32_t tq_sel;          // landmark-only pass: 64-query tiles (selection rows) per head
};

// Byte offset of 16-byte chunk `chunk` of 128-byte row `row` in a tile. The
// chunk index is XORed with a function of the row chosen so that both MFMA
// operand reads are bank-conflict free on gfx950's LDS: the K read (16 lanes
// on 16 consecutive rows, same chunk) and the transposed V read (4
// consecutive rows, 64 contiguous bytes each).
__device__ __forceinline__ int swz_f(int row) { return (((row >> 1) & 1) << 2) | ((row >> 2) & 3); }
__device__ __forceinline__ uint32_t swz(int row, int chunk) {
  return (uint32_t)(row * 128 + ((chunk ^ swz_f(row)) << 4));
}

// Workgroup barrier without the memory fence of __syncthreads(): that fence
// waits for every outstanding vector-memory op, including the direct-to-LDS
// loads still in flight. LDS reads are complete (lgkmcnt) first; the loads of
// the blocks about to be read are waited for explicitly (vmcnt).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// The value must be computed at this point of the program (an empty asm
// that reads it); keeps the compiler from sinking its computation further.
template <typename T>
__device__ __forceinline__ void keep_vgpr(T x) {
  asm volatile("" ::"v"(x));
}

// 16 bytes per lane from a buffer resource straight into LDS (the buffer
// form of the direct-to-LDS load: reads past the records return zeros)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kBufferFlags);
}
__device__ __forceinline__ void buffer_to_lds(__amdgpu_buffer_rsrc_t r,
                                              __attribute__((address_space(3))) void* dst,
                                              uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, 0, 0, 0);
}
// f(integral_constant<int, 0>) ... f(integral_constant<int, N - 1>), in order
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(static_cast<F&&>(f));
  }
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0f70 | (N & 15) | ((N >> 4) << 14));
}

__device__ __forceinline__ float sum8_sq(u32x4 w) {
  float s = 0.f;
  const uint32_t e[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = bf16lo(e[i]), b = bf16hi(e[i]);
    s = __builtin_fmaf(a, a, s);
    s = __builtin_fmaf(b, b, s);
  }
  return s;
}

__device__ __forceinline__ float max8_abs(u32x4 w) {
  const uint32_t m = 0x7fff7fffu;  // clear both sign bits
  const uint32_t e[4] = {w.x & m, w.y & m, w.z & m, w.w & m};
  float r = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) r = fmaxf(r, fmaxf(bf16lo(e[i]), bf16hi(e[i])));
  return r;
}

// Partial maxima of |k|^2 over key rows and landmark rows, and of |v| over
// value and landmark-value entries: part[h][c] for chunk c of each row set.
__global__ __launch_bounds__(256) void range_kernel(const uint16_t* __restrict__ k,
                                                    const uint16_t* __restrict__ v, int64_t nk,
                                                    int64_t kst, int64_t ksh,
                                                    const uint16_t* __restrict__ kb,
                                                    const uint16_t* __restrict__ vb, int32_t tk,
                                                    float* __restrict__ part) {
  __shared__ float red[2][4];
  const int c = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int sub = tid & 7;  // 16-byte chunk of a row
  const int rl = tid >> 3;  // one of 32 rows per pass
  float k2 = 0.f, vm = 0.f;
  auto rows = [&](const uint16_t* kp, const uint16_t* vp, int64_t n, int64_t st) {
    const int64_t per = (n + kRangeParts - 1) / kRangeParts;
    const int64_t r0 = (int64_t)c * per, r1 = min(n, r0 + per);
    // the 8 lanes of one row share the trip count, so the shuffles stay in step
    for (int64_t r = r0 + rl; r < r1; r += 32) {
      const u32x4 kw = *(const u32x4*)(kp + r * st + 8 * sub);
      const u32x4 vw = *(const u32x4*)(vp + r * st + 8 * sub);
      float s = sum8_sq(kw);
      s += __shfl_xor(s, 1, kWave);
      s += __shfl_xor(s, 2, kWave);
      s += __shfl_xor(s, 4, kWave);
      k2 = fmaxf(k2, s);
      vm = fmaxf(vm, max8_abs(vw));
    }
  };
  rows(k + (int64_t)h * ksh, v + (int64_t)h * ksh, nk, kst);
  if (kb != nullptr)
    rows(kb + (int64_t)h * tk * kHeadDim, vb + (int64_t)h * tk * kHeadDim, tk, kHeadDim);
  k2 = wave_max(k2);
  vm = wave_max(vm);
  if ((tid & 63) == 0) {
    red[0][tid >> 6] = k2;
    red[1][tid >> 6] = vm;
  }
  __syncthreads();
  if (tid == 0) {
    float* out = part + ((int64_t)h * kRangeParts + c) * 2;
    out[0] = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
    out[1] = fmaxf(fmaxf(red[1][0], red[1][1]), fmaxf(red[1][2], red[1][3]));
  }
}

template <int QT, int KT>
__global__ __launch_bounds__(QT * 2) __attribute__((amdgpu_waves_per_eu(QT >= 64 ? 2 : 1))) void tile_sparse_kernel(SparseParams p,
                                                             const int32_t* __restrict__ sel) {
  constexpr int W = QT / 32;             // waves
  constexpr int NT = W * kWave;          // threads
  constexpr int NB = KT / 32;            // 32-key score blocks per tile
  constexpr int TILE_BYTES = KT * 128;   // one K (or V) block in LDS
  constexpr int KB_PER_TILE = TILE_BYTES / 1024;  // 1 KB direct-to-LDS wave loads
  constexpr int NU = KB_PER_TILE / W;    // 1 KB blocks per wave per tensor
  static_assert(KB_PER_TILE % W == 0, "load split");

  // Two-stage K and V rings. Distinct LDS objects, indexed with compile-time
  // stage numbers, let the compiler prove that reads of one stage do not
  // alias the direct-to-LDS writes in flight to another, so it adds no waits
  // for those loads before LDS reads.
  __shared__ u32x4 ks0[KB_PER_TILE][64], ks1[KB_PER_TILE][64];
  __shared__ u32x4 vs0[KB_PER_TILE][64], vs1[KB_PER_TILE][64];
  __shared__ uint16_t win[kWin];             // window of the kept list
  __shared__ uint32_t kept_bits[kBitWords];  // kept key tiles of the item
  __shared__ int32_t slow_item;
  typedef __attribute__((address_space(3))) u32x4 lds_blk[64];
  auto kbuf = [&](auto stc) -> lds_blk* {
    if constexpr (decltype(stc)::value == 0) return (lds_blk*)ks0;
    else return (lds_blk*)ks1;
  };
  auto vbuf = [&](auto stc) -> lds_blk* {
    if constexpr (decltype(stc)::value == 0) return (lds_blk*)vs0;
    else return (lds_blk*)vs1;
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // uniform per wave
  const int lane = tid % kWave;
  const int qi = lane & 31;  // query within the wave / column of S^T
  const int hh = lane >> 5;  // lane half
  const bool dense = sel == nullptr;
  const int n_lb_all = dense || !p.landmarks ? 0 : (p.tk + KT - 1) / KT;  // landmark blocks
  const int tail_rows = (int)(p.nk - (int64_t)(p.tk - 1) * KT);  // rows of tile tk-1
  const int last_lrows = p.tk - (n_lb_all - 1) * KT;  // landmark rows in the last block
  const float c = p.scale_log2;
  const bool log_count = p.log_count != 0;
  const float lm_shift = log_count ? p.lm_log2_kt : 0.f;  // landmark columns, log2 units
  const int n_ch = p.n_chunks;
  const int lb_per_chunk = p.chunk_tiles / KT;
  const int64_t items_per_head = (int64_t)n_ch * p.tq;

  // ---- direct-to-LDS staging. 1 KB block u of a tile holds rows 8u..8u+7;
  // lane i writes physical chunk i%8 of row r = 8u + i/8, i.e. logical chunk
  // (i%8) ^ swz_f(r). This wave stages blocks u = wave + W v.
  // Per-lane byte offsets of the MFMA operand reads within a staged block
  // (the same for every item). K: key row qi, chunk 2s + hh; the second score
  // block is 32 rows (4096 bytes) further. V (transposed reads): lane group
  // G = lane/16 covers channel offset 16(G%2) and key half G/2; each of the
  // two reads returns 4 consecutive keys (rows r0 and r0 + 8) of the lane's
  // channel, channel block db adds 32 channels; each further 16 keys are 16
  // rows (2048 bytes) further. The swizzle depends on row bits 1-3 only, so
  // those row steps are plain offsets.
  uint32_t koff[4], voff[2][2];
#pragma unroll
  for (int s = 0; s < 4; ++s) koff[s] = swz(qi, 2 * s + hh);
  {
    const int G = lane >> 4, S = lane & 15;
    const int r0 = 4 * (G >> 1) + (S >> 2);
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      const int col = 32 * db + 16 * (G & 1) + 4 * (S & 3);
      const int chunk = col >> 3, half = (col & 7) ? 8 : 0;
      voff[db][0] = swz(r0, chunk) + half;
      voff[db][1] = swz(r0 + 8, chunk) + half;
    }
  }
  const int lrow = lane >> 3;
  int lchunk[NU];
  uint32_t off_kv[NU], off_lm[NU];
#pragma unroll
  for (int v = 0; v < NU; ++v) {
    const int r = 8 * (wave + W * v) + lrow;
    lchunk[v] = (lane & 7) ^ swz_f(r);
    off_kv[v] = (uint32_t)(r * p.kst * 2 + lchunk[v] * 16);
    off_lm[v] = (uint32_t)(r * 128 + lchunk[v] * 16);
  }

  for (int64_t item = blockIdx.x; item < p.n_items; item += gridDim.x) {
    const int h = (int)(item / items_per_head);
    const int64_t rem = item - (int64_t)h * items_per_head;
    const int ch = (int)(rem / p.tq);
    const int qtile = (int)(rem - (int64_t)ch * p.tq);
    const int64_t row = (int64_t)h * p.tq + qtile;  // (head, query tile)
    // the item's kept entries [kept0, kept0 + n_kept) and landmark blocks [lb0, lb0 + n_lb)
    int kept0 = 0, n_kept = dense ? p.tk : p.top_k, lb0 = 0, n_lb = n_lb_all;
    if (n_ch > 1) {
      const int32_t* co = p.coff + row * (n_ch + 1) + ch;
      kept0 = __builtin_amdgcn_readfirstlane(co[0]);
      n_kept = max(__builtin_amdgcn_readfirstlane(co[1]) - kept0, 0);
      lb0 = ch * lb_per_chunk;
      n_lb = n_lb_all > 0 ? min(lb_per_chunk, n_lb_all - lb0) : 0;
    }
    const int n_total = n_kept + n_lb;
    const int32_t* sel_row = dense ? nullptr : sel + row * p.top_k + kept0;
    const uint8_t* kh = (const uint8_t*)(p.k + (int64_t)h * p.ksh);
    const uint8_t* vh = (const uint8_t*)(p.v + (int64_t)h * p.ksh);
    const bool has_lm = n_lb_all > 0;
    const uint8_t* klm =
        has_lm ? (const uint8_t*)(p.kbar_b + (int64_t)h * p.tk * kHeadDim) : nullptr;
    const uint8_t* vlm =
        has_lm ? (const uint8_t*)(p.vbar_b + (int64_t)h * p.tk * kHeadDim) : nullptr;

    lds_barrier();  // every wave is done with the previous item's LDS
    if (tid == 0) slow_item = 0;
    if (n_lb > 0) {
      const int words = NB * n_lb;  // every word the item's landmark blocks read
      for (int e = tid; e < words; e += NT) kept_bits[NB * lb0 + e] = 0u;
    }
    if (!dense) {
      const int nw = min(kWin, n_kept);
      for (int e = tid; e < nw; e += NT) win[e] = (uint16_t)min(max(sel_row[e], 0), p.tk - 1);
    }
    // query operand (B of S^T = K Q^T): Q[q][16s + 8hh .. +7]
    const int64_t qrow = (int64_t)qtile * QT + wave * 32 + qi;
    const bool qvalid = qrow < p.nq;
    bf16x8 qop[4];
    float qq = 0.f;
    {
      const uint16_t* qp = p.q + (int64_t)h * p.qsh + qrow * p.qst + 8 * hh;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        u32x4 w = {0u, 0u, 0u, 0u};
        if (qvalid) w = *(const u32x4*)(qp + 16 * s);
        qop[s] = as_bf16x8(w);
        qq += sum8_sq(w);
      }
    }
    float k2 = p.range[((int64_t)h * kRangeParts + lane) * 2];
    float vmax = p.range[((int64_t)h * kRangeParts + lane) * 2 + 1];
    const int last_kept =
        dense ? p.tk - 1 : (n_kept > 0 ? min(max(sel_row[n_kept - 1], 0), p.tk - 1) : -1);
    __syncthreads();  // also completes every vector load above
    if (n_lb > 0)
      for (int e = tid; e < n_kept; e += NT) {
        const int j = min(max(sel_row[e], 0), p.tk - 1);
        atomicOr(&kept_bits[j >> 5], 1u << (j & 31));
      }
    k2 = wave_max(k2);
    vmax = wave_max(vmax);
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(qq), __float_as_uint(qq),
                                                       false, false);
      qq = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);  // own half + partner half
    }
    // upper bound of this query's logits in log2 units (relative margin for
    // the float32 products, sums and square roots)
    const float m_q =
        c * __builtin_sqrtf(qq) * __builtin_sqrtf(k2) * (1.0f + 1.0f / 64.0f) + 1.0f;
    const bool fast_ok = m_q <= kBoundLimit && vmax <= kVLimit;
    if (!__all(fast_ok) && lane == 0) slow_item = 1;
    __syncthreads();  // bitmap and vote complete (and the sel loads drained)
    const bool fast = slow_item == 0;
    const int last_rows = last_kept == p.tk - 1 ? tail_rows : KT;

    // ---- the item's block list through the rings
    int win_lo = 0;
    // collective; makes kept entries t_v <= t_k (those below n_kept) readable
    auto ensure_window = [&](int t_v, int t_k) {
      if (dense || t_v >= n_kept) return;
      const int hi = min(t_k, n_kept - 1);
      if (t_v >= win_lo && hi < win_lo + kWin) return;
      win_lo = t_v;
      const int nw = min(kWin, n_kept - t_v);
      for (int e = tid; e < nw; e += NT)
        win[e] = (uint16_t)min(max(sel_row[t_v + e], 0), p.tk - 1);
      __syncthreads();  // no direct-to-LDS load is in flight here
    };
    auto dma = [&](const void* src, lds_blk* dst, int u) {
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)&dst[u][0],
                                       16, 0, 0);
    };
    // sources of block t of the list: kept key tile (rows past a short last
    // tile repeat its last row) or landmark block (rows past tk repeat row
    // tk-1); this wave's 1 KB pieces v = 0..NU-1 go to blocks wave + W v
    struct Src {
      const uint8_t* base;
      uint32_t off[NU];
    };
    auto prep = [&](int t, const uint8_t* th, const uint8_t* tl) -> Src {
      const uint8_t* base;
      uint32_t off[NU];
      int rows;
      int64_t row_bytes;
      if (t < n_kept) {
        const int j = dense ? t : __builtin_amdgcn_readfirstlane(win[t - win_lo]);
        base = th + (int64_t)j * KT * p.kst * 2;
        rows = j == p.tk - 1 ? tail_rows : KT;
        row_bytes = p.kst * 2;
#pragma unroll
        for (int v = 0; v < NU; ++v) off[v] = off_kv[v];
      } else {
        const int b = lb0 + t - n_kept;
        base = tl + (int64_t)b * KT * 128;
        rows = b == n_lb_all - 1 ? last_lrows : KT;
        row_bytes = 128;
#pragma unroll
        for (int v = 0; v < NU; ++v) off[v] = off_lm[v];
      }
      if (rows < KT) {  // rare: rows past the end repeat the last valid row
#pragma unroll
        for (int v = 0; v < NU; ++v) {
          const int r = min(8 * (wave + W * v) + lrow, rows - 1);
          off[v] = (uint32_t)(r * row_bytes + lchunk[v] * 16);
        }
      }
      Src src;
      src.base = base;
#pragma unroll
      for (int v = 0; v < NU; ++v) src.off[v] = off[v];
      return src;
    };
    auto fire = [&](const Src& src, lds_blk* dst, int v) {
      dma(src.base + src.off[v], dst, wave + W * v);
    };
    auto issue = [&](int t, const uint8_t* th, const uint8_t* tl, lds_blk* dst) {
      const Src src = prep(t, th, tl);
#pragma unroll
      for (int v = 0; v < NU; ++v) fire(src, dst, v);
    };
    // excluded columns of block t (bit set = excluded), or 0
    auto block_mask = [&](int t) -> uint64_t {
      if (t < n_kept) return t == n_kept - 1 && last_rows < KT ? ~0ull << last_rows : 0ull;
      const int b = lb0 + t - n_kept;
      const uint32_t lo = __builtin_amdgcn_readfirstlane(kept_bits[NB * b]);
      const uint32_t hi = KT == 64 ? __builtin_amdgcn_readfirstlane(kept_bits[2 * b + 1]) : 0u;
      uint64_t m = ((uint64_t)hi << 32) | lo;
      if (b == n_lb_all - 1 && last_lrows < KT) m |= ~0ull << last_lrows;
      return m;
    };

    // ---- products
    // K operands of one block (A of S^T = K Q^T): ka[b][s] = K[32b + qi][16s + 8hh .. +7]
    auto read_k1 = [&](auto kst_c, bf16x8 (&ka)[NB][4], int b, int s) {
      const lds_u8* ks = (const lds_u8*)kbuf(kst_c);
      ka[b][s] =
          as_bf16x8(*(const __attribute__((address_space(3))) u32x4*)(ks + koff[s] + 4096 * b));
    };
    auto read_k = [&](auto kst_c, bf16x8 (&ka)[NB][4]) {
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int s = 0; s < 4; ++s) read_k1(kst_c, ka, b, s);
    };
    auto qk_b = [&](const bf16x8 (&ka)[NB][4], f32x16& sacc, int b) {
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[b][0], qop[0], f32x16{}, 0, 0, 0);
#pragma unroll
      for (int s = 1; s < 4; ++s) sacc = mfma32(ka[b][s], qop[s], sacc);
    };
    f32x16 oacc[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      oacc[0][i] = 0.f;
      oacc[1][i] = 0.f;
    }
    // V operands (A of O^T[d][q] += V^T[d][key] P^T[key][q]), 16 keys per
    // MFMA. va[m][db]: keys 16m.., channels 32db..
    auto read_v = [&](auto vst_c, u32x4 (&va)[2 * NB][2], int m_lo, int m_hi) {
      const lds_u8* vs = (const lds_u8*)vbuf(vst_c);
#pragma unroll
      for (int m = m_lo; m < m_hi; ++m)
#pragma unroll
        for (int db = 0; db < 2; ++db) {
          const i16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4*)(vs + voff[db][0] + 2048 * m));
          const i16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4*)(vs + voff[db][1] + 2048 * m));
          const u32x2 w0 = __builtin_bit_cast(u32x2, t0), w1 = __builtin_bit_cast(u32x2, t1);
          va[m][db] = u32x4{w0.x, w0.y, w1.x, w1.y};
        }
    };
    auto pv_m = [&](const u32x4 (&va)[2 * NB][2], bf16x8 pop, int m) {
#pragma unroll
      for (int db = 0; db < 2; ++db) oacc[db] = mfma32(as_bf16x8(va[m][db]), pop, oacc[db]);
    };
    const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3f803f80u);
    float l_run = 0.f;
    float mc_run = -INFINITY;  // fallback: running maximum in log2 units
    const float nm_fast = kPShift - m_q - lm_shift;
    // lane holds keys 32b + 8g + 4hh + r in register 4g + r of score block b.
    // colmask is uniform: per register, the excluded lanes form a 64-bit lane
    // mask built with scalar ops, applied by one v_cndmask.
    // register i of score block b holds key 32b + 8(i/4) + 4hh + i%4: the
    // lanes (half hh = 0: low 32, hh = 1: high 32) whose key is set in the
    // uniform column mask, as a 64-bit lane mask (two sign-extended bits)
    auto lanes_of = [&](uint64_t colmask, int b, int i) -> uint64_t {
      const uint32_t w = (uint32_t)(colmask >> (32 * b));
      const int off = 8 * (i >> 2) + (i & 3);
      const uint32_t lo = (uint32_t)(((int32_t)(w << (31 - off))) >> 31);
      const uint32_t hi = (uint32_t)(((int32_t)(w << (27 - off))) >> 31);
      return ((uint64_t)hi << 32) | lo;
    };
    auto apply_mask = [&](f32x16 (&sacc)[NB], uint64_t colmask) {
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (__builtin_amdgcn_inverse_ballot_w64(lanes_of(colmask, b, i))) sacc[b][i] = -INFINITY;
    };
    // probabilities of one score block -> two PV operands, row sum updated
    auto probs = [&](const f32x16& s, float nm, bf16x8& lo8, bf16x8& hi8) {
      uint32_t w[8];
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c, nm));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i + 1], c, nm));
        w[i >> 1] = pack_bf16x2(p0, p1);
        l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[i >> 1]), ones,
                                                l_run, false);
      }
      lo8 = as_bf16x8(u32x4{w[0], w[1], w[2], w[3]});
      hi8 = as_bf16x8(u32x4{w[4], w[5], w[6], w[7]});
    };
    // one pair of probabilities (registers 2i, 2i+1 of a score block) as a
    // packed bf16 word; row sum updated
    auto prob_pair = [&](const f32x16& s, int i, float nm) -> uint32_t {
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * i], c, nm));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * i + 1], c, nm));
      const uint32_t w = pack_bf16x2(p0, p1);
      l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), ones, l_run, false);
      return w;
    };
    // fallback: running maximum with lazy rescale of l; returns -reference.
    // When the reference moves, alpha (per lane) is the factor that O takes
    // once the pending PV product of the previous block is in, and the return
    // flag (uniform) says so.
    auto online_ref = [&](const f32x16 (&sacc)[NB], float& nm, float& alpha) -> bool {
      float tm0 = sacc[0][0], tm1 = sacc[0][1];
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = (b == 0 ? 2 : 0); i < 16; i += 2) {
          tm0 = __builtin_elementwise_maximum(tm0, sacc[b][i]);
          tm1 = __builtin_elementwise_maximum(tm1, sacc[b][i + 1]);
        }
      float tmax = __builtin_elementwise_maximum(tm0, tm1);
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax),
                                                       __float_as_uint(tmax), false, false);
      tmax = __builtin_elementwise_maximum(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      const float tmc = tmax * c;
      bool moved = false;
      alpha = 1.f;
      if (__any(tmc > mc_run + kRescaleSlack)) {
        const float m_new = __builtin_elementwise_maximum(mc_run, tmc);
        alpha = __builtin_amdgcn_exp2f(mc_run - m_new);
        l_run *= alpha;
        mc_run = m_new;
        moved = true;
      }
      nm = -mc_run;
      return moved;
    };

    // variant V2: the landmark of the short last key tile counts its tail_rows
    // tokens, not KT: add corr to the score of column col (uniform) of the block,
    // with the same uniform lane masks as apply_mask
    auto add_col = [&](f32x16 (&sacc)[NB], int col, float corr) {
      const uint64_t m = 1ull << col;
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (__builtin_amdgcn_inverse_ballot_w64(lanes_of(m, b, i))) sacc[b][i] += corr;
    };

    // S(t) of the current block; P of the last two blocks (bf16 PV operands),
    // indexed by block parity. P(-1) = 0, so the PV step of block -1 adds
    // nothing.
    f32x16 sacc[NB];
    bf16x8 pb0[2 * NB], pb1[2 * NB];
#pragma unroll
    for (int m = 0; m < 2 * NB; ++m) pb1[m] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
    auto pbuf = [&](auto par) -> bf16x8(&)[2 * NB] {
      if constexpr (decltype(par)::value == 0) return pb0;
      else return pb1;
    };

    // One step t (parity par = t & 1): wait for K(t+1) and V(t-1), issue
    // K(t+2) into K stage par and V(t) into V stage par, then the softmax of
    // block t (S(t) -> P(t)) interleaved with PV(t-1), then QK(t+1). The
    // first two steps (t = -2, -1) only fill the rings and compute QK(0); a
    // last PV step follows the loop. Every step issues the same number of
    // loads (past either end of the list the nearest block is loaded again),
    // so the outstanding-load count the waits rely on is exact.
    auto run = [&](auto fast_c) {
      constexpr bool kFast = decltype(fast_c)::value;
      auto body = [&](auto par, auto masked_c, uint64_t cmask, float nm_add, int tail_col) {
        constexpr bool kMasked = decltype(masked_c)::value;
        using R = std::integral_constant<int, 1 - decltype(par)::value>;
        u32x4 va[2 * NB][2];
        bf16x8 ka[NB][4];
        read_v(R{}, va, 0, 2);  // V(t-1), first 32 keys
        read_k(R{}, ka);        // K(t+1); past the end a repeated block
        if constexpr (kMasked) {
          if (tail_col >= 0) add_col(sacc, tail_col, p.lm_tail_corr);
          apply_mask(sacc, cmask);
        }
        float nm = nm_fast, alpha = 1.f;
        bool moved = false;
        if constexpr (!kFast) moved = online_ref(sacc, nm, alpha);
        if constexpr (kMasked) nm += nm_add;  // landmark blocks: log2(KT) under V2
        bf16x8(&pw)[2 * NB] = pbuf(par);
        bf16x8(&pr)[2 * NB] = pbuf(R{});
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          if (b == 1) read_v(R{}, va, 2, 4);  // V(t-1), last 32 keys
          probs(sacc[b], nm, pw[2 * b], pw[2 * b + 1]);
          pv_m(va, pr[2 * b], 2 * b);
          pv_m(va, pr[2 * b + 1], 2 * b + 1);
        }
        if constexpr (!kFast) {
          if (moved) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              oacc[0][i] *= alpha;
              oacc[1][i] *= alpha;
            }
          }
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) qk_b(ka, sacc[b], b);  // QK(t+1)
        // P(t) and the row sum are complete within this step (keeps the
        // compiler from sinking the softmax into the next step, past its barrier)
#pragma unroll
        for (int m = 0; m < 2 * NB; ++m)
          keep_vgpr(__builtin_bit_cast(u32x4, pw[m]));
        keep_vgpr(l_run);
      };
      // The fast step of 64-key blocks with the instruction order fixed
      // by scheduling fences: 16 MFMA slots, and the 16 pair jobs (two
      // probabilities each) spread over the first 12 so that each wave's
      // MFMAs run while it issues its own softmax arithmetic. Two jobs while
      // the operand reads land; slots 1-8: PV(t-1) (P(t-1) and V(t-1) are
      // ready), one job each; slots 9-12: QK(t+1) into score block 0 (its
      // probabilities are out), the last six jobs; 13-16: QK(t+1) into score
      // block 1.
      auto body_fast64 = [&](auto par, auto masked_c, uint64_t cmask, float nm_add,
                             int tail_col, const Src& sk, const Src& sv) {
        if constexpr (KT == 64) {
          using R = std::integral_constant<int, 1 - decltype(par)::value>;
          u32x4 va[4][2];
          bf16x8 ka[2][4];
          uint32_t w0[8], w1[8];
          bf16x8(&pw)[4] = pbuf(par);
          bf16x8(&pr)[4] = pbuf(R{});
          float nm = nm_fast;
          read_v(R{}, va, 0, 2);  // V(t-1), first 32 keys
          if constexpr (decltype(masked_c)::value) {
            if (tail_col >= 0) add_col(sacc, tail_col, p.lm_tail_corr);
            apply_mask(sacc, cmask);
            nm += nm_add;  // landmark blocks: log2(KT) under V2
          }
          // pair jobs in order: score block 0 pairs 0-7, then block 1 pairs 0-7
          auto job = [&](int n) {
            if (n < 8)
              w0[n] = prob_pair(sacc[0], n, nm);
            else
              w1[n - 8] = prob_pair(sacc[1], n - 8, nm);
          };
          job(0);  // while the operand reads land
          job(1);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int j = 0; j < 8; ++j) {  // slots 1-8: PV(t-1), jobs 2-9
            oacc[j & 1] = mfma32(as_bf16x8(va[j >> 1][j & 1]), pr[j >> 1], oacc[j & 1]);
            job(2 + j);
            // the other operand reads, at most 15 in flight: K(t+1) of score
            // block 0 (slots 1-2), V(t-1) of the last 32 keys (3-4), K(t+1)
            // of score block 1 (5-6); past the end a repeated block
            if (j < 2 || (j >= 4 && j < 6)) {
              read_k1(R{}, ka, j >> 2, 2 * (j & 1));
              read_k1(R{}, ka, j >> 2, 2 * (j & 1) + 1);
            }
            if (j == 2 || j == 3) read_v(R{}, va, j, j + 1);
            // the loads of K(t+2) and V(t): 2 NU pieces over slots 1-8
            constexpr int kPer = (2 * NU + 7) / 8;
#pragma unroll
            for (int k = 0; k < kPer; ++k) {
              const int q = j * kPer + k;
              if (q < NU)
                fire(sk, kbuf(par), q);
              else if (q < 2 * NU)
                fire(sv, vbuf(par), q - NU);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
          pw[0] = as_bf16x8(u32x4{w0[0], w0[1], w0[2], w0[3]});
          pw[1] = as_bf16x8(u32x4{w0[4], w0[5], w0[6], w0[7]});
#pragma unroll
          for (int j = 0; j < 4; ++j) {  // slots 9-12: QK(t+1) of score block 0, jobs 10-15
            sacc[0] = j == 0 ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[0][0], qop[0], f32x16{},
                                                                        0, 0, 0)
                             : mfma32(ka[0][j], qop[j], sacc[0]);
            job(10 + (j < 2 ? 2 * j : j + 2));
            if (j < 2) job(11 + 2 * j);
            __builtin_amdgcn_sched_barrier(0);
          }
          pw[2] = as_bf16x8(u32x4{w1[0], w1[1], w1[2], w1[3]});
          pw[3] = as_bf16x8(u32x4{w1[4], w1[5], w1[6], w1[7]});
          qk_b(ka, sacc[1], 1);  // slots 13-16
#pragma unroll
          for (int m = 0; m < 4; ++m) keep_vgpr(__builtin_bit_cast(u32x4, pw[m]));
          keep_vgpr(l_run);
        }
      };
      // masked_c: the block may exclude columns (landmark blocks and a short
      // last kept tile); the other blocks run the branch-free body
      auto step = [&](int t, auto par, auto masked_c) {
        wait_vmcnt<0>();  // this wave's loads of K(t+1), V(t-1) have landed
        lds_barrier();    // ... and every other wave's; stage par of both rings is free
        const int tkn = min(t + 2, n_total - 1);
        const int tvn = max(min(t, n_total - 1), 0);
        ensure_window(tvn, tkn);
        const Src sk = prep(tkn, kh, klm), sv = prep(tvn, vh, vlm);
        // the fast 64-key steps issue these loads inside their MFMA slots
        constexpr bool kSpread = kFast && KT == 64;
        if (!kSpread || t < 0) {
#pragma unroll
          for (int v = 0; v < NU; ++v) fire(sk, kbuf(par), v);
#pragma unroll
          for (int v = 0; v < NU; ++v) fire(sv, vbuf(par), v);
        }
        if (t == -1) {
          bf16x8 ka[NB][4];
          read_k(P0{}, ka);
#pragma unroll
          for (int b = 0; b < NB; ++b) qk_b(ka, sacc[b], b);  // QK(0)
        }
        if (t < 0) return;
        if constexpr (decltype(masked_c)::value) {
          const bool lm = t >= n_kept;
          const int tcol = lm && log_count && lb0 + t - n_kept == n_lb_all - 1 && tail_rows < KT
                               ? last_lrows - 1
                               : -1;
          if constexpr (kFast && KT == 64)
            body_fast64(par, masked_c, block_mask(t), lm ? lm_shift : 0.f, tcol, sk, sv);
          else
            body(par, masked_c, block_mask(t), lm ? lm_shift : 0.f, tcol);
        } else if constexpr (kFast && KT == 64) {
          body_fast64(par, masked_c, 0ull, 0.f, -1, sk, sv);
        } else {
          body(par, masked_c, 0ull, 0.f, -1);
        }
      };
      // PV of the last block t = n_total - 1 (parity par)
      auto drain = [&](auto par) {
        wait_vmcnt<0>();  // also: no direct-to-LDS load outlives the item
        lds_barrier();
        u32x4 va[2 * NB][2];
        read_v(par, va, 0, 2 * NB);
        bf16x8(&pr)[2 * NB] = pbuf(par);
#pragma unroll
        for (int m = 0; m < 2 * NB; ++m) pv_m(va, pr[m], m);
      };
      using Plain = std::false_type;
      using Masked = std::true_type;
      // blocks [0, n_plain) need no column mask
      const int n_plain = last_rows < KT ? n_kept - 1 : n_kept;
      step(-2, P0{}, Plain{});
      step(-1, P1{}, Plain{});
      int t = 0;
      for (; t + 2 <= n_plain; t += 2) {
        step(t, P0{}, Plain{});
        step(t + 1, P1{}, Plain{});
      }
      if (t < n_plain) step(t++, P0{}, Plain{});
      if ((t & 1) && t < n_total) step(t++, P1{}, Masked{});
      for (; t + 2 <= n_total; t += 2) {
        step(t, P0{}, Masked{});
        step(t + 1, P1{}, Masked{});
      }
      if (t < n_total) step(t, P0{}, Masked{});
      if ((n_total - 1) & 1)
        drain(P1{});
      else
        drain(P0{});
    };
    if (n_total > 0) {  // an item may have no columns: split keys without landmarks
      if (fast)
        run(std::true_type{});
      else
        run(std::false_type{});
    }

    // ---- epilogue: O / l, lane (qi, hh) holds channels 32db + 8g + 4hh + r
    const auto lsw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run),
                                                      __float_as_uint(l_run), false, false);
    const float l_sum = __uint_as_float(lsw[0]) + __uint_as_float(lsw[1]);
    if (n_ch > 1) {  // split keys: unnormalised partial and (reference, row sum)
      if (qvalid) {
        const int64_t prow = ((int64_t)h * p.nq + qrow) * p.part_slots + ch;
        float* op = p.part_o + prow * kHeadDim + 4 * hh;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g)
            *(f32x4*)(op + 32 * db + 8 * g) = f32x4{oacc[db][4 * g], oacc[db][4 * g + 1],
                                                    oacc[db][4 * g + 2], oacc[db][4 * g + 3]};
        if (hh == 0) p.part_ml[prow] = float2{fast ? -nm_fast : mc_run, l_sum};
      }
      continue;
    }
    if (p.lse != nullptr && qvalid && hh == 0)
      p.lse[(int64_t)h * p.nq + qrow] = (fast ? -nm_fast : mc_run) + __builtin_log2f(l_sum);
    const float inv = 1.0f / l_sum;
    if (qvalid) {
      if (p.o_f32) {
        float* op = (float*)p.o + (int64_t)h * p.osh + qrow * p.ost + 4 * hh;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            f32x4 w = {oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv,
                       oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv};
            *(f32x4*)(op + 32 * db + 8 * g) = w;
          }
      } else {
        uint16_t* op = (uint16_t*)p.o + (int64_t)h * p.osh + qrow * p.ost + 4 * hh;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            u32x2 w = {pack_bf16x2(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv),
                       pack_bf16x2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv)};
            *(u32x2*)(op + 32 * db + 8 * g) = w;
          }
      }
    }
  }
}

// Key-half decomposition (64-key tiles; 64 or 128 queries per item, i.e. 2
// or 4 waves). Wave w takes key half kh = w % 2 (keys 32kh .. 32kh + 31 of
// every block) for query group qg = w / 2 (64 queries, two 32-query MFMA
// column tiles qh = 0, 1). Every K or V operand fragment read from LDS then
// feeds two MFMAs, one per query half: half the LDS operand traffic of the
// one-wave-per-32-queries layout, the other large user of LDS bandwidth
// besides the direct-to-LDS loads. Rings, block list and pipeline are those
// of tile_sparse_kernel. At the end of an item the two key halves of a query
// group meet in LDS: wave kh keeps query half kh and hands the other half's
// partial output, row sum and reference to its partner. With the fixed
// reference both partials share it and simply add; on the fallback path each
// is first scaled to the larger of the two running maxima.
// The second query group's kept-tile bitmap of the landmark-only pass
// (function-local, so only that instantiation holds it in LDS).
__device__ __forceinline__ uint32_t* lm_bits_second() {
  __shared__ uint32_t bits[kBitWords];
  return bits;
}

// kLmOnly (128-query tiles, split keys): an item is one (head, pair of 64-query
// tiles) over every landmark block of the head, query group qg masked by the
// kept tiles of 64-query tile 2 g + qg. It runs after the key-chunk launch and
// merges its landmark columns' unnormalised output and (reference, row sum)
// with the chunks' partials of its queries, in slot order with its own last,
// into the normalised output (and the normaliser when asked for).
template <int QT, bool kLmOnly>
__global__ __launch_bounds__(QT * 2) __attribute__((amdgpu_waves_per_eu(2))) void tile_sparse_kh_kernel(
    SparseParams p, const int32_t* __restrict__ sel) {
  constexpr int KT = 64;
  constexpr int W = QT / 32;             // waves: (query group, key half) pairs
  constexpr int NT = W * kWave;
  constexpr int KB_PER_TILE = KT * 128 / 1024;
  constexpr int NU = KB_PER_TILE / W;    // 1 KB direct-to-LDS pieces per wave per tensor
  static_assert(KB_PER_TILE % W == 0 && W >= 2, "load split");
  static_assert(!kLmOnly || QT == 128, "landmark-only items are 128-query pairs");

  __shared__ u32x4 ks0[KB_PER_TILE][64], ks1[KB_PER_TILE][64];
  __shared__ u32x4 vs0[KB_PER_TILE][64], vs1[KB_PER_TILE][64];
  __shared__ uint16_t win[kWin];
  __shared__ uint32_t kept_bits[kBitWords];
  __shared__ int32_t slow_item;
  typedef __attribute__((address_space(3))) u32x4 lds_blk[64];
  auto kbuf = [&](auto stc) -> lds_blk* {
    if constexpr (decltype(stc)::value == 0) return (lds_blk*)ks0;
    else return (lds_blk*)ks1;
  };
  auto vbuf = [&](auto stc) -> lds_blk* {
    if constexpr (decltype(stc)::value == 0) return (lds_blk*)vs0;
    else return (lds_blk*)vs1;
  };
  // end-of-item exchange: wave w's 8 KB of partial output in ring block w
  // (the lane's slot address is formed where it is used: an empty asm hides
  // the uniform base from loop-invariant code motion, which would otherwise
  // keep one address per slot live across the item loop)
  auto xbuf = [&](int w) -> __attribute__((address_space(3))) f32x4* {
    u32x4* b = w == 0 ? &ks0[0][0] : (w == 1 ? &ks1[0][0] : (w == 2 ? &vs0[0][0] : &vs1[0][0]));
    uint32_t a = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) u32x4*)b;
    asm volatile("" : "+s"(a));
    return (__attribute__((address_space(3))) f32x4*)(uintptr_t)a;
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int kh = wave & 1, qg = wave >> 1;
  const int lane = tid % kWave;
  const int qi = lane & 31;
  const int hh = lane >> 5;
  const bool dense = sel == nullptr;
  const int n_lb_all = dense || !p.landmarks ? 0 : (p.tk + KT - 1) / KT;
  const int tail_rows = (int)(p.nk - (int64_t)(p.tk - 1) * KT);
  const int last_lrows = p.tk - (n_lb_all - 1) * KT;
  const float c = p.scale_log2;
  const bool log_count = p.log_count != 0;
  const float lm_shift = log_count ? p.lm_log2_kt : 0.f;
  const int n_ch = p.n_chunks;
  const int lb_per_chunk = p.chunk_tiles / KT;
  const int64_t items_per_head = (int64_t)n_ch * p.tq;

  // Operand read offsets within a staged block (see tile_sparse_kernel); the
  // key half adds 32 rows (4096 bytes).
  uint32_t koff[4], voff[2][2];
#pragma unroll
  for (int s = 0; s < 4; ++s) koff[s] = swz(qi, 2 * s + hh) + 4096 * kh;
  {
    const int G = lane >> 4, S = lane & 15;
    const int r0 = 4 * (G >> 1) + (S >> 2);
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      const int col = 32 * db + 16 * (G & 1) + 4 * (S & 3);
      const int chunk = col >> 3, half = (col & 7) ? 8 : 0;
      voff[db][0] = swz(r0, chunk) + half + 4096 * kh;
      voff[db][1] = swz(r0 + 8, chunk) + half + 4096 * kh;
    }
  }
  // direct-to-LDS staging as in tile_sparse_kernel, through buffer
  // resources; the resource of a block ends at its last valid row, so the
  // rows past a short last tile read as zeros (their columns are masked).
  // With two waves each wave stages exactly its own key half (pieces
  // 4 kh .. 4 kh + 3, rows 32 kh ..), so no wave reads what another loaded
  // and the steps need no workgroup barrier, only the wave's own waits.
  // With four waves piece v of wave w is w + 4 v and the steps synchronise
  // the workgroup. Piece u covers rows 8 u + lane / 8, lane chunk
  // (lane % 8) ^ swz_f(row).
  constexpr bool kOwnHalf = W == 2;
  // blocks in flight ahead of use: with own-half staging a wave refills the
  // ring stage it has just read (its own rows only) with the blocks two steps
  // ahead, once its reads of that stage have completed; with four waves the
  // stages are shared and each is refilled one step ahead behind a barrier
  constexpr int kAhead = kOwnHalf ? 2 : 1;
  const int lrow = lane >> 3;
  auto piece = [&](int v) { return kOwnHalf ? 4 * kh + v : wave + W * v; };
  // (key/value rows are 128 bytes apart here, like landmark rows)
  uint32_t off_v[NU];
#pragma unroll
  for (int v = 0; v < NU; ++v) {
    const int r = 8 * piece(v) + lrow;
    off_v[v] = (uint32_t)(r * 128 + (((lane & 7) ^ swz_f(r)) << 4));
  }
  // end of a step's waits: with own-half staging the wave's own loads and
  // LDS reads; otherwise also every other wave's
  auto step_sync = [&]() {
    if constexpr (kOwnHalf)
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    else
      lds_barrier();
  };

  for (int64_t item = blockIdx.x; item < p.n_items; item += gridDim.x) {
    // per-item copies of the argument pointers that lane addresses are formed
    // from: hidden from loop-invariant code motion, which would hoist one
    // 64-bit address per lane out of the item loop and spill it
    const uint16_t* q_arg = p.q;
    const float* range_arg = p.range;
    void* o_arg = p.o;
    float* part_o_arg = p.part_o;
    asm volatile("" : "+s"(q_arg), "+s"(range_arg), "+s"(o_arg), "+s"(part_o_arg));
    const int h = (int)(item / (kLmOnly ? (int64_t)p.tq : items_per_head));
    const int64_t rem = item - (int64_t)h * (kLmOnly ? (int64_t)p.tq : items_per_head);
    const int ch = kLmOnly ? p.part_slots - 1 : (int)(rem / p.tq);
    const int qtile = kLmOnly ? (int)rem : (int)(rem - (int64_t)ch * p.tq);
    const int64_t row = (int64_t)h * p.tq + qtile;
    int kept0 = 0, n_kept = dense ? p.tk : p.top_k, lb0 = 0, n_lb = n_lb_all;
    if constexpr (kLmOnly) {
      n_kept = 0;  // every landmark block, masked per query group below
    } else if (n_ch > 1) {
      const int32_t* co = p.coff + row * (n_ch + 1) + ch;
      kept0 = __builtin_amdgcn_readfirstlane(co[0]);
      n_kept = max(__builtin_amdgcn_readfirstlane(co[1]) - kept0, 0);
      lb0 = ch * lb_per_chunk;
      // (only two-wave items hand their landmark blocks to the separate pass)
      n_lb = n_lb_all > 0 && !(kOwnHalf && p.lm_separate) ? min(lb_per_chunk, n_lb_all - lb0) : 0;
    }
    // the selection rows of the pair's two 64-query tiles (landmark-only pass)
    const int64_t lm_row0 = (int64_t)h * p.tq_sel + min(2 * qtile, p.tq_sel - 1);
    const int64_t lm_row1 = (int64_t)h * p.tq_sel + min(2 * qtile + 1, p.tq_sel - 1);
    // this wave's kept-tile bitmap (its query group's, in the landmark-only pass)
    uint32_t* my_bits = kept_bits;
    if constexpr (kLmOnly) my_bits = qg == 0 ? kept_bits : lm_bits_second();
    const int n_total = n_kept + n_lb;
    const int32_t* sel_row = dense ? nullptr : sel + row * p.top_k + kept0;
    // Walk order of the kept list. Any order gives the same softmax up to
    // rounding; with a phase period P (the items the device runs at once) the
    // walk starts at the first kept tile at or after position (item mod P) / P
    // of the item's key range and wraps around. Items are dispatched in index
    // order at a steady rate, P at a time, so the items in flight walk the
    // same part of the range together and share its blocks in L2. A short
    // last key tile stays the last step, where its missing rows are masked.
    // (Two-wave items only: split keys run them.)
    int rot = 0, n_rot = 0;
    if (kOwnHalf && !dense && p.phase_period > 0 && n_kept > 1) {
      const int last = __builtin_amdgcn_readfirstlane(sel_row[n_kept - 1]);
      n_rot = (last >= p.tk - 1 && tail_rows < KT) ? n_kept - 1 : n_kept;
      const int span = n_ch > 1 ? p.chunk_tiles : p.tk;
      const int target = (n_ch > 1 ? ch * p.chunk_tiles : 0) +
                         (int)((item % p.phase_period) * span / p.phase_period);
      int lo = 0, hi = n_rot;  // first entry >= target (the list ascends)
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (__builtin_amdgcn_readfirstlane(sel_row[mid]) < target)
          lo = mid + 1;
        else
          hi = mid;
      }
      rot = lo < n_rot ? lo : 0;
    }
    auto kept_at = [&](int e) -> uint16_t {
      int i = e;
      if constexpr (kOwnHalf) {
        if (e < n_rot) {
          i = e + rot;
          if (i >= n_rot) i -= n_rot;
        }
      }
      return (uint16_t)min(max(sel_row[i], 0), p.tk - 1);
    };
    const uint8_t* khp = (const uint8_t*)(p.k + (int64_t)h * p.ksh);
    const uint8_t* vhp = (const uint8_t*)(p.v + (int64_t)h * p.ksh);
    const bool has_lm = n_lb_all > 0;
    const uint8_t* klm =
        has_lm ? (const uint8_t*)(p.kbar_b + (int64_t)h * p.tk * kHeadDim) : nullptr;
    const uint8_t* vlm =
        has_lm ? (const uint8_t*)(p.vbar_b + (int64_t)h * p.tk * kHeadDim) : nullptr;

    lds_barrier();  // every wave is done with the previous item's LDS
    if (tid == 0) slow_item = 0;
    if (n_lb > 0) {
      const int words = 2 * n_lb;
      for (int e = tid; e < words; e += NT) kept_bits[2 * lb0 + e] = 0u;
      if constexpr (kLmOnly)
        for (int e = tid; e < words; e += NT) lm_bits_second()[e] = 0u;
    }
    if (!dense) {
      const int nw = min(kWin, n_kept);
      for (int e = tid; e < nw; e += NT) win[e] = kept_at(e);
    }
    // query operands of both query halves: Q[q][16s + 8hh .. +7]
    const int64_t qbase = (int64_t)qtile * QT + 64 * qg + qi;
    bf16x8 qop[2][4];
    float qq[2] = {0.f, 0.f};
#pragma unroll
    for (int qh = 0; qh < 2; ++qh) {
      const int64_t qr = qbase + 32 * qh;
      const uint16_t* qp = q_arg + (int64_t)h * p.qsh + qr * p.qst + 8 * hh;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        u32x4 w = {0u, 0u, 0u, 0u};
        if (qr < p.nq) w = *(const u32x4*)(qp + 16 * s);
        qop[qh][s] = as_bf16x8(w);
        qq[qh] += sum8_sq(w);
      }
    }
    float k2 = range_arg[((int64_t)h * kRangeParts + lane) * 2];
    float vmax = range_arg[((int64_t)h * kRangeParts + lane) * 2 + 1];
    const int last_kept =
        dense ? p.tk - 1 : (n_kept > 0 ? min(max(sel_row[n_kept - 1], 0), p.tk - 1) : -1);
    __syncthreads();
    if constexpr (kLmOnly) {
      // eight loads in flight per lane before the first bit is set
      const int n2 = 2 * p.top_k;
      for (int e0 = tid; e0 < n2; e0 += 8 * NT) {
        int jv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int e = min(e0 + u * NT, n2 - 1);
          const int g = e >= p.top_k;
          jv[u] = sel[(g ? lm_row1 : lm_row0) * p.top_k + e - g * p.top_k];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int e = e0 + u * NT;
          if (e < n2) {
            const int j = min(max(jv[u], 0), p.tk - 1);
            atomicOr(&(e >= p.top_k ? lm_bits_second() : kept_bits)[j >> 5], 1u << (j & 31));
          }
        }
      }
    } else if (n_lb > 0) {
      for (int e = tid; e < n_kept; e += NT) {
        const int j = min(max(sel_row[e], 0), p.tk - 1);
        atomicOr(&kept_bits[j >> 5], 1u << (j & 31));
      }
    }
    k2 = wave_max(k2);
    vmax = wave_max(vmax);
    float m_q[2], nm_fast[2];
    bool fast_ok = vmax <= kVLimit;
#pragma unroll
    for (int qh = 0; qh < 2; ++qh) {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(qq[qh]),
                                                       __float_as_uint(qq[qh]), false, false);
      const float q2 = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      m_q[qh] = c * __builtin_sqrtf(q2) * __builtin_sqrtf(k2) * (1.0f + 1.0f / 64.0f) + 1.0f;
      fast_ok = fast_ok && m_q[qh] <= kBoundLimit;
      nm_fast[qh] = kPShift - m_q[qh] - lm_shift;
    }
    if (!__all(fast_ok) && lane == 0) slow_item = 1;
    __syncthreads();
    const bool fast = slow_item == 0;
    const int last_rows = last_kept == p.tk - 1 ? tail_rows : KT;

    int win_lo = 0;
    auto ensure_window = [&](int t_v, int t_k) {
      if (dense || t_v >= n_kept) return;
      const int hi = min(t_k, n_kept - 1);
      if (t_v >= win_lo && hi < win_lo + kWin) return;
      // the waves may be at different steps (own-half staging): every wave
      // has passed its reads of the old window first
      __syncthreads();
      win_lo = t_v;
      const int nw = min(kWin, n_kept - t_v);
      for (int e = tid; e < nw; e += NT) win[e] = kept_at(t_v + e);
      __syncthreads();  // no direct-to-LDS load is in flight here
    };
    // a block as a buffer resource whose records end at its last valid row
    typedef __amdgpu_buffer_rsrc_t Src;
    auto prep = [&](int t, const uint8_t* th, const uint8_t* tl) -> Src {
      const uint8_t* base;
      int rows;
      if (t < n_kept) {
        const int j = dense ? t : __builtin_amdgcn_readfirstlane(win[t - win_lo]);
        rows = j == p.tk - 1 ? tail_rows : KT;
        base = th + (int64_t)j * KT * 128;
      } else {
        const int b = lb0 + t - n_kept;
        rows = b == n_lb_all - 1 ? last_lrows : KT;
        base = tl + (int64_t)b * KT * 128;
      }
      return block_rsrc(base, rows * 128);
    };
    auto fire = [&](const Src& src, lds_blk* dst, auto v_c) {
      constexpr int v = decltype(v_c)::value;
      buffer_to_lds(src, (__attribute__((address_space(3))) void*)&dst[piece(v)][0], off_v[v]);
    };
    auto block_mask = [&](int t) -> uint64_t {
      if (t < n_kept) return t == n_kept - 1 && last_rows < KT ? ~0ull << last_rows : 0ull;
      const int b = lb0 + t - n_kept;
      const uint32_t lo = __builtin_amdgcn_readfirstlane(my_bits[2 * b]);
      const uint32_t hi = __builtin_amdgcn_readfirstlane(my_bits[2 * b + 1]);
      uint64_t m = ((uint64_t)hi << 32) | lo;
      if (b == n_lb_all - 1 && last_lrows < KT) m |= ~0ull << last_lrows;
      return m;
    };

    // ---- products (this wave's 32 keys of a block; both query halves)
    auto read_k1 = [&](auto kst_c, bf16x8 (&ka)[4], int s) {
      const lds_u8* ks = (const lds_u8*)kbuf(kst_c);
      ka[s] = as_bf16x8(*(const __attribute__((address_space(3))) u32x4*)(ks + koff[s]));
    };
    auto read_v = [&](auto vst_c, u32x4 (&va)[2][2]) {
      const lds_u8* vs = (const lds_u8*)vbuf(vst_c);
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int db = 0; db < 2; ++db) {
          const i16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4*)(vs + voff[db][0] + 2048 * m));
          const i16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4*)(vs + voff[db][1] + 2048 * m));
          const u32x2 w0 = __builtin_bit_cast(u32x2, t0), w1 = __builtin_bit_cast(u32x2, t1);
          va[m][db] = u32x4{w0.x, w0.y, w1.x, w1.y};
        }
    };
    f32x16 oacc[2][2];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      oacc[0][0][i] = 0.f;
      oacc[0][1][i] = 0.f;
      oacc[1][0][i] = 0.f;
      oacc[1][1][i] = 0.f;
    }
    auto qk_q = [&](const bf16x8 (&ka)[4], f32x16& sacc, int qh) {
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[0], qop[qh][0], f32x16{}, 0, 0, 0);
#pragma unroll
      for (int s = 1; s < 4; ++s) sacc = mfma32(ka[s], qop[qh][s], sacc);
    };
    const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3f803f80u);
    float l_run[2] = {0.f, 0.f};
    float mc_run[2] = {-INFINITY, -INFINITY};
    // register i holds key 32kh + 8(i/4) + 4hh + i%4 of the block
    auto lanes_of = [&](uint32_t w, int i) -> uint64_t {
      const int off = 8 * (i >> 2) + (i & 3);
      const uint32_t lo = (uint32_t)(((int32_t)(w << (31 - off))) >> 31);
      const uint32_t hi = (uint32_t)(((int32_t)(w << (27 - off))) >> 31);
      return ((uint64_t)hi << 32) | lo;
    };
    auto apply_mask = [&](f32x16 (&sacc)[2], uint64_t colmask) {
      const uint32_t w = (uint32_t)(colmask >> (32 * kh));
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const bool ex = __builtin_amdgcn_inverse_ballot_w64(lanes_of(w, i));
        if (ex) {
          sacc[0][i] = -INFINITY;
          sacc[1][i] = -INFINITY;
        }
      }
    };
    // Fixed-reference path: the excluded columns of S(t) take one more MFMA step
    // per query half, the rank-one product of a key-side operand holding -2^100
    // (exact in bf16) in the excluded key rows and 0 elsewhere with a query-side
    // operand of ones. Kept scores gain exactly 0; excluded ones fall to about
    // -2^100, whose probability 2^(c s - m_q + 60) is 0, as -inf gives. Four VALU
    // instructions per block instead of a select per score register.
    const bf16x8 ones_k0 = as_bf16x8(u32x4{lane < 32 ? 0x3f80u : 0u, 0u, 0u, 0u});
    auto mask_by_mfma = [&](f32x16 (&sacc)[2], uint64_t colmask) {
      const uint32_t w = (uint32_t)(colmask >> (32 * kh));
      const uint32_t ex = lane < 32 ? (w >> qi) & 1u : 0u;
      const bf16x8 big = as_bf16x8(u32x4{ex != 0u ? 0xf180u : 0u, 0u, 0u, 0u});
      sacc[0] = mfma32(big, ones_k0, sacc[0]);
      sacc[1] = mfma32(big, ones_k0, sacc[1]);
    };
    auto add_col = [&](f32x16 (&sacc)[2], int col, float corr) {
      const int lc = col - 32 * kh;
      if (lc < 0 || lc >= 32) return;  // uniform
      const uint32_t w = 1u << lc;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (__builtin_amdgcn_inverse_ballot_w64(lanes_of(w, i))) {
          sacc[0][i] += corr;
          sacc[1][i] += corr;
        }
    };
    auto prob_pair = [&](const f32x16& s, int i, float nm, float& l) -> uint32_t {
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * i], c, nm));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * i + 1], c, nm));
      const uint32_t w = pack_bf16x2(p0, p1);
      l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), ones, l, false);
      return w;
    };
    // fallback: running maximum per query half with lazy rescale of l;
    // returns whether any reference moved (alpha then scales O after the
    // pending PV product)
    auto online_ref = [&](const f32x16 (&sacc)[2], float (&nm)[2], float (&alpha)[2]) -> bool {
      bool moved_any = false;
      float tmc[2];
#pragma unroll
      for (int qh = 0; qh < 2; ++qh) {
        float tm0 = sacc[qh][0], tm1 = sacc[qh][1];
#pragma unroll
        for (int i = 2; i < 16; i += 2) {
          tm0 = __builtin_elementwise_maximum(tm0, sacc[qh][i]);
          tm1 = __builtin_elementwise_maximum(tm1, sacc[qh][i + 1]);
        }
        float tmax = __builtin_elementwise_maximum(tm0, tm1);
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax),
                                                         __float_as_uint(tmax), false, false);
        tmax = __builtin_elementwise_maximum(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        tmc[qh] = tmax * c;
      }
      if (__any(tmc[0] > mc_run[0] + kRescaleSlack || tmc[1] > mc_run[1] + kRescaleSlack)) {
#pragma unroll
        for (int qh = 0; qh < 2; ++qh) {
          const float m_new = __builtin_elementwise_maximum(mc_run[qh], tmc[qh]);
          alpha[qh] = __builtin_amdgcn_exp2f(mc_run[qh] - m_new);
          l_run[qh] *= alpha[qh];
          mc_run[qh] = m_new;
        }
        moved_any = true;
      }
      // a key half can see only excluded columns so far (a short last block):
      // any finite shift then gives them probability zero
      nm[0] = mc_run[0] == -INFINITY ? 0.f : -mc_run[0];
      nm[1] = mc_run[1] == -INFINITY ? 0.f : -mc_run[1];
      return moved_any;
    };

    // S(t) of both query halves; P of the last two blocks by block parity,
    // pb[qh][m] = keys 16m.. of this wave's half
    f32x16 sacc[2];
    bf16x8 pb0[2][2], pb1[2][2];
#pragma unroll
    for (int qh = 0; qh < 2; ++qh)
#pragma unroll
      for (int m = 0; m < 2; ++m) pb1[qh][m] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
    auto pbuf = [&](auto par) -> bf16x8(&)[2][2] {
      if constexpr (decltype(par)::value == 0) return pb0;
      else return pb1;
    };

    auto run = [&](auto fast_c) {
      constexpr bool kFast = decltype(fast_c)::value;
      // One step: softmax of block t (both query halves, 16 pair jobs) with
      // PV(t-1) (8 MFMAs), then QK(t+1) (8 MFMAs). The fast path fixes the
      // order with scheduling fences: two jobs while the operand reads land,
      // slots 1-8 PV(t-1) with one job each, slots 9-12 QK(t+1) of query
      // half 0 with the last six jobs, slots 13-16 QK(t+1) of query half 1;
      // the loads of K(t+2) and V(t) go out in slots 1-8.
      auto body = [&](auto par, auto masked_c, uint64_t cmask, float nm_add, int tail_col,
                      const Src& sk, const Src& sv) {
        constexpr bool kMasked = decltype(masked_c)::value;
        using R = std::integral_constant<int, 1 - decltype(par)::value>;
        u32x4 va[2][2];
        bf16x8 ka[4];
        uint32_t w[2][8];
        bf16x8(&pw)[2][2] = pbuf(par);
        bf16x8(&pr)[2][2] = pbuf(R{});
        read_v(R{}, va);  // V(t-1)
        if constexpr (kAhead == 2) {
          // K(t+1) too: stage R is refilled below once both reads are done
#pragma unroll
          for (int s = 0; s < 4; ++s) read_k1(R{}, ka, s);
        }
        if constexpr (kMasked) {
          if (tail_col >= 0) add_col(sacc, tail_col, p.lm_tail_corr);
          if constexpr (kFast && !kOwnHalf)
            mask_by_mfma(sacc, cmask);
          else
            apply_mask(sacc, cmask);
        }
        float nm[2] = {nm_fast[0], nm_fast[1]}, alpha[2] = {1.f, 1.f};
        bool moved = false;
        if constexpr (!kFast) moved = online_ref(sacc, nm, alpha);
        if constexpr (kMasked) {
          nm[0] += nm_add;
          nm[1] += nm_add;
        }
        auto job = [&](int n) {
          const int qh = n >> 3, i = n & 7;
          w[qh][i] = prob_pair(sacc[qh], i, nm[qh], l_run[qh]);
        };
        job(0);
        job(1);
        if constexpr (kFast) __builtin_amdgcn_sched_barrier(0);
        static_for<8>([&](auto jc) {  // slots 1-8: PV(t-1)
          constexpr int j = decltype(jc)::value;
          constexpr int qh = j >> 2, m = (j >> 1) & 1, db = j & 1;
          oacc[qh][db] = mfma32(as_bf16x8(va[m][db]), pr[qh][m], oacc[qh][db]);
          job(2 + j);
          if constexpr (kAhead == 2) {
            // K(t+3) and V(t+1) into stage R, whose reads (V(t-1), K(t+1))
            // must have completed first: an LDS write by a global load is not
            // ordered after LDS reads still in flight
            if constexpr (j == 2) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            static_assert(NU == 4, "own-half staging: 4 pieces per tensor");
            constexpr int q0 = j < 2 ? 8 : (j < 4 ? 2 * (j - 2) : j);
            constexpr int nq = j < 2 ? 0 : (j < 4 ? 2 : 1);
            static_for<nq>([&](auto kc) {
              constexpr int q = q0 + decltype(kc)::value;
              if constexpr (q < NU)
                fire(sk, kbuf(R{}), std::integral_constant<int, q>{});
              else
                fire(sv, vbuf(R{}), std::integral_constant<int, q - NU>{});
            });
          } else {
            if constexpr (j < 2) {
              read_k1(R{}, ka, 2 * j);  // K(t+1); past the end a repeated block
              read_k1(R{}, ka, 2 * j + 1);
            }
            constexpr int kPer = (2 * NU + 7) / 8;
            static_for<kPer>([&](auto kc) {
              constexpr int q = j * kPer + decltype(kc)::value;
              if constexpr (q < NU)
                fire(sk, kbuf(par), std::integral_constant<int, q>{});
              else if constexpr (q < 2 * NU)
                fire(sv, vbuf(par), std::integral_constant<int, q - NU>{});
            });
          }
          if constexpr (kFast) __builtin_amdgcn_sched_barrier(0);
        });
        if constexpr (!kFast) {
          if (moved) {
#pragma unroll
            for (int qh = 0; qh < 2; ++qh)
#pragma unroll
              for (int db = 0; db < 2; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) oacc[qh][db][i] *= alpha[qh];
          }
        }
        pw[0][0] = as_bf16x8(u32x4{w[0][0], w[0][1], w[0][2], w[0][3]});
        pw[0][1] = as_bf16x8(u32x4{w[0][4], w[0][5], w[0][6], w[0][7]});
#pragma unroll
        for (int j = 0; j < 4; ++j) {  // slots 9-12: QK(t+1) of query half 0
          sacc[0] = j == 0 ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[0], qop[0][0], f32x16{},
                                                                      0, 0, 0)
                           : mfma32(ka[j], qop[0][j], sacc[0]);
          job(10 + (j < 2 ? 2 * j : j + 2));
          if (j < 2) job(11 + 2 * j);
          if constexpr (kFast) __builtin_amdgcn_sched_barrier(0);
        }
        pw[1][0] = as_bf16x8(u32x4{w[1][0], w[1][1], w[1][2], w[1][3]});
        pw[1][1] = as_bf16x8(u32x4{w[1][4], w[1][5], w[1][6], w[1][7]});
        qk_q(ka, sacc[1], 1);  // slots 13-16
        // P(t) and the row sums are complete within this step
#pragma unroll
        for (int qh = 0; qh < 2; ++qh)
#pragma unroll
          for (int m = 0; m < 2; ++m) keep_vgpr(__builtin_bit_cast(u32x4, pw[qh][m]));
        keep_vgpr(l_run[0]);
        keep_vgpr(l_run[1]);
      };
      auto step = [&](int t, auto par, auto masked_c) {
        // the blocks read in this step were issued kAhead steps ago; the
        // kAhead - 1 newer steps' loads (2 NU each) may stay in flight
        wait_vmcnt<2 * NU * (kAhead - 1)>();
        step_sync();
        if constexpr (decltype(masked_c)::value == 2) {
          // streaming step: 0 <= t < n_kept - 2 - kAhead, so K(t + 1 + kAhead)
          // and V(t + kAhead - 1) are whole kept tiles (the short last tile is
          // at most the last kept one) and the whole kept list is in the window
          const int jk = dense ? t + 1 + kAhead
                               : __builtin_amdgcn_readfirstlane(win[t + 1 + kAhead]);
          const int jv = dense ? t + kAhead - 1
                               : __builtin_amdgcn_readfirstlane(win[t + kAhead - 1]);
          const Src sk = block_rsrc(khp + (int64_t)jk * (KT * 128), KT * 128);
          const Src sv = block_rsrc(vhp + (int64_t)jv * (KT * 128), KT * 128);
          body(par, std::false_type{}, 0ull, 0.f, -1, sk, sv);
        } else if constexpr (decltype(masked_c)::value == 3) {
          // landmark streaming step: n_kept <= t < n_total - 2 - kAhead, so
          // block t and the loaded blocks K(t + 1 + kAhead), V(t + kAhead - 1)
          // are whole landmark blocks (the head's last one, which may be short
          // or carry the log-count correction, is the item's last block)
          const int b = lb0 + t - n_kept;
          const Src sk = block_rsrc(klm + (int64_t)(b + 1 + kAhead) * (KT * 128), KT * 128);
          const Src sv = block_rsrc(vlm + (int64_t)(b + kAhead - 1) * (KT * 128), KT * 128);
          const uint32_t lo = __builtin_amdgcn_readfirstlane(my_bits[2 * b]);
          const uint32_t hi = __builtin_amdgcn_readfirstlane(my_bits[2 * b + 1]);
          body(par, std::true_type{}, ((uint64_t)hi << 32) | lo, lm_shift, -1, sk, sv);
        } else {
        const int tkn = min(t + 1 + kAhead, n_total - 1);
        const int tvn = max(min(t + kAhead - 1, n_total - 1), 0);
        ensure_window(tvn, tkn);
        const Src sk = prep(tkn, khp, klm), sv = prep(tvn, vhp, vlm);
        if (t < 0) {
          static_for<NU>([&](auto vc) { fire(sk, kbuf(par), vc); });
          static_for<NU>([&](auto vc) { fire(sv, vbuf(par), vc); });
        }
        if (t == -1) {
          bf16x8 ka[4];
#pragma unroll
          for (int s = 0; s < 4; ++s) read_k1(P0{}, ka, s);
          qk_q(ka, sacc[0], 0);  // QK(0)
          qk_q(ka, sacc[1], 1);
        }
        if (t < 0) return;
        if constexpr (decltype(masked_c)::value == 1) {
          const bool lm = t >= n_kept;
          const int tcol = lm && log_count && lb0 + t - n_kept == n_lb_all - 1 && tail_rows < KT
                               ? last_lrows - 1
                               : -1;
          body(par, masked_c, block_mask(t), lm ? lm_shift : 0.f, tcol, sk, sv);
        } else {
          body(par, masked_c, 0ull, 0.f, -1, sk, sv);
        }
        }
      };
      auto drain = [&](auto par) {  // PV of the last block
        wait_vmcnt<0>();
        step_sync();
        u32x4 va[2][2];
        read_v(par, va);
        bf16x8(&pr)[2][2] = pbuf(par);
#pragma unroll
        for (int qh = 0; qh < 2; ++qh)
#pragma unroll
          for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int db = 0; db < 2; ++db)
              oacc[qh][db] = mfma32(as_bf16x8(va[m][db]), pr[qh][m], oacc[qh][db]);
      };
      using Plain = std::false_type;
      using Masked = std::true_type;
      const int n_plain = last_rows < KT ? n_kept - 1 : n_kept;
      using Stream = std::integral_constant<int, 2>;
      // streaming steps need the whole kept list in the window (then it
      // starts at entry 0 and never moves)
      const int n_stream = (dense || n_kept <= kWin) ? max(n_kept - 2 - kAhead, 0) : 0;
      if constexpr (kAhead == 2) {
        // K(0) -> stage 0, K(1) -> stage 1, and V(0) -> V stage 1 as a finite
        // stand-in for the absent V(-1) (its probabilities P(-1) are zero);
        // QK(0) once K(0) has landed; then K(2) -> stage 0 and V(0) -> V stage 0
        ensure_window(0, min(2, n_total - 1));
        const Src k0 = prep(0, khp, klm), k1 = prep(min(1, n_total - 1), khp, klm);
        const Src v0 = prep(0, vhp, vlm);
        static_for<NU>([&](auto vc) { fire(k0, kbuf(P0{}), vc); });
        static_for<NU>([&](auto vc) { fire(k1, kbuf(P1{}), vc); });
        static_for<NU>([&](auto vc) { fire(v0, vbuf(P1{}), vc); });
        wait_vmcnt<2 * NU>();
        bf16x8 ka[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) read_k1(P0{}, ka, s);
        qk_q(ka, sacc[0], 0);  // QK(0)
        qk_q(ka, sacc[1], 1);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        const Src k2 = prep(min(2, n_total - 1), khp, klm);
        static_for<NU>([&](auto vc) { fire(k2, kbuf(P0{}), vc); });
        static_for<NU>([&](auto vc) { fire(v0, vbuf(P0{}), vc); });
      } else {
        step(-2, P0{}, Plain{});
        step(-1, P1{}, Plain{});
      }
      int t = 0;
      for (; t + 2 <= n_stream; t += 2) {
        step(t, P0{}, Stream{});
        step(t + 1, P1{}, Stream{});
      }
      for (; t + 2 <= n_plain; t += 2) {
        step(t, P0{}, Plain{});
        step(t + 1, P1{}, Plain{});
      }
      if (t < n_plain) step(t++, P0{}, Plain{});
      if ((t & 1) && t < n_total) step(t++, P1{}, Masked{});
      // (the landmark-only pass: in the other items the extra step form costs
      // the register allocation more than it saves)
      if constexpr (kLmOnly) {
        using LmStream = std::integral_constant<int, 3>;
        const int n_lms = n_lb > 0 ? n_total - 2 - kAhead : 0;
        for (; t + 2 <= n_lms; t += 2) {  // (no kept tiles: t >= n_kept = 0)
          step(t, P0{}, LmStream{});
          step(t + 1, P1{}, LmStream{});
        }
      }
      for (; t + 2 <= n_total; t += 2) {
        step(t, P0{}, Masked{});
        step(t + 1, P1{}, Masked{});
      }
      if (t < n_total) step(t, P0{}, Masked{});
      if ((n_total - 1) & 1)
        drain(P1{});
      else
        drain(P0{});
    };
    if (n_total > 0) {
      if (fast)
        run(std::true_type{});
      else
        run(std::false_type{});
    }

    // ---- merge the key halves. Row sums over the lane halves first.
    float l_q[2], ref_q[2];
#pragma unroll
    for (int qh = 0; qh < 2; ++qh) {
      const auto lsw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run[qh]),
                                                        __float_as_uint(l_run[qh]), false, false);
      l_q[qh] = __uint_as_float(lsw[0]) + __uint_as_float(lsw[1]);
      ref_q[qh] = fast ? -nm_fast[qh] : mc_run[qh];
    }
    // wave kh keeps query half kh and hands over query half 1 - kh: its
    // partial output (lane-major f32x4 slots) and per-query (reference, sum)
    lds_barrier();  // every wave is done with the rings
    // (kh is uniform: both branches index the register arrays statically)
    auto put = [&](const f32x16 (&og)[2], float r, float l) {
      __attribute__((address_space(3))) f32x4* xb = xbuf(wave);
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          xb[(db * 4 + g) * 64 + lane] =
              f32x4{og[db][4 * g], og[db][4 * g + 1], og[db][4 * g + 2], og[db][4 * g + 3]};
      float2* xm = (float2*)win;  // 32 (reference, sum) pairs per wave
      if (hh == 0) xm[wave * 32 + qi] = float2{r, l};
    };
    if (kh == 0)
      put(oacc[1], ref_q[1], l_q[1]);
    else
      put(oacc[0], ref_q[0], l_q[0]);
    __syncthreads();
    // merge into the kept half's accumulators and write the query half kh
    auto finish = [&](f32x16 (&om)[2], float r_mine, float l_mine) {
      const int partner = wave ^ 1;
      const __attribute__((address_space(3))) f32x4* xb = xbuf(partner);
      const float2 pm = ((const float2*)win)[partner * 32 + qi];
      float ref = __builtin_elementwise_maximum(r_mine, pm.x);
      // a partial without columns (l = 0) carries no weight
      const float a_mine = l_mine > 0.f ? __builtin_amdgcn_exp2f(r_mine - ref) : 0.f;
      const float a_part = pm.y > 0.f ? __builtin_amdgcn_exp2f(pm.x - ref) : 0.f;
      const float l_sum = l_mine * a_mine + pm.y * a_part;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 x = xb[(db * 4 + g) * 64 + lane];
#pragma unroll
          for (int r = 0; r < 4; ++r)
            om[db][4 * g + r] = om[db][4 * g + r] * a_mine + x[r] * a_part;
        }
      if (l_sum == 0.f) ref = r_mine;  // no columns at all (split keys, no landmarks)
      const int64_t qrow = qbase + 32 * kh;
      if (qrow >= p.nq) return;
      if constexpr (kLmOnly) {
        // The key chunks' partials of this query are complete (the pass runs
        // after the chunk launch, on the same stream): merge them with this
        // one, which is the last slot, exactly as the combine does: reference
        // R = the largest over the partials with columns, then in slot order
        // l = sum l_c 2^(r_c - R) and O = sum O_c 2^(r_c - R), then O / l.
        const int64_t prow0 = ((int64_t)h * p.nq + qrow) * p.part_slots;
        const float2* ml = p.part_ml + prow0;
        const float* po = part_o_arg + prow0 * kHeadDim + 4 * hh;
        float big = l_sum > 0.f ? ref : -INFINITY;
        for (int c = 0; c < n_ch; ++c) {
          const float2 m = ml[c];
          if (m.y > 0.f) big = __builtin_elementwise_maximum(big, m.x);
        }
        float l_tot = 0.f;
        f32x4 acc[2][4];
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) acc[db][g] = f32x4{0.f, 0.f, 0.f, 0.f};
        auto add = [&](float2 m, const f32x4 (&x)[2][4]) {
          const float wgt = m.y > 0.f ? __builtin_amdgcn_exp2f(m.x - big) : 0.f;
          l_tot = __builtin_fmaf(m.y, wgt, l_tot);
#pragma unroll
          for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g)
#pragma unroll
              for (int r = 0; r < 4; ++r)
                acc[db][g][r] = __builtin_fmaf(x[db][g][r], wgt, acc[db][g][r]);
        };
        for (int c = 0; c < n_ch; ++c) {
          f32x4 x[2][4];
#pragma unroll
          for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g)
              x[db][g] = *(const f32x4*)(po + (int64_t)c * kHeadDim + 32 * db + 8 * g);
          add(ml[c], x);
        }
        {
          f32x4 x[2][4];
#pragma unroll
          for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g)
              x[db][g] = f32x4{om[db][4 * g], om[db][4 * g + 1], om[db][4 * g + 2],
                               om[db][4 * g + 3]};
          add(float2{ref, l_sum}, x);
        }
        const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;  // 0 only without any column
        if (p.lse != nullptr && hh == 0)
          p.lse[(int64_t)h * p.nq + qrow] = big + __builtin_log2f(l_tot);
        if (p.o_f32) {
          float* op = (float*)o_arg + (int64_t)h * p.osh + qrow * p.ost + 4 * hh;
#pragma unroll
          for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g)
              *(f32x4*)(op + 32 * db + 8 * g) =
                  f32x4{acc[db][g][0] * inv, acc[db][g][1] * inv, acc[db][g][2] * inv,
                        acc[db][g][3] * inv};
        } else {
          uint16_t* op = (uint16_t*)o_arg + (int64_t)h * p.osh + qrow * p.ost + 4 * hh;
#pragma unroll
          for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g)
              *(u32x2*)(op + 32 * db + 8 * g) =
                  u32x2{pack_bf16x2(acc[db][g][0] * inv, acc[db][g][1] * inv),
                        pack_bf16x2(acc[db][g][2] * inv, acc[db][g][3] * inv)};
        }
        return;
      }
      if (n_ch > 1) {  // split keys: unnormalised partial, (reference, row sum)
        // (four-wave key-chunk items are never split: their stride stays n_ch)
        const int slots = kOwnHalf ? p.part_slots : n_ch;
        const int64_t prow = ((int64_t)h * p.nq + qrow) * slots + ch;
        float* op = part_o_arg + prow * kHeadDim + 4 * hh;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g)
            *(f32x4*)(op + 32 * db + 8 * g) =
                f32x4{om[db][4 * g], om[db][4 * g + 1], om[db][4 * g + 2], om[db][4 * g + 3]};
        if (hh == 0) p.part_ml[prow] = float2{ref, l_sum};
        return;
      }
      if (p.lse != nullptr && hh == 0)
        p.lse[(int64_t)h * p.nq + qrow] = ref + __builtin_log2f(l_sum);
      const float inv = 1.0f / l_sum;
      if (p.o_f32) {
        float* op = (float*)o_arg + (int64_t)h * p.osh + qrow * p.ost + 4 * hh;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g)
            *(f32x4*)(op + 32 * db + 8 * g) =
                f32x4{om[db][4 * g] * inv, om[db][4 * g + 1] * inv, om[db][4 * g + 2] * inv,
                      om[db][4 * g + 3] * inv};
      } else {
        uint16_t* op = (uint16_t*)o_arg + (int64_t)h * p.osh + qrow * p.ost + 4 * hh;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            u32x2 w = {pack_bf16x2(om[db][4 * g] * inv, om[db][4 * g + 1] * inv),
                       pack_bf16x2(om[db][4 * g + 2] * inv, om[db][4 * g + 3] * inv)};
            *(u32x2*)(op + 32 * db + 8 * g) = w;
          }
      }
    };
    if (kh == 0)
      finish(oacc[0], ref_q[0], l_q[0]);
    else
      finish(oacc[1], ref_q[1], l_q[1]);
  }
}

// fp32 landmarks -> bf16 rows [H][tk][64].
__global__ void pack_landmarks_kernel(const float* __restrict__ kbar,
                                      const float* __restrict__ vbar, int64_t n_pairs,
                                      uint16_t* __restrict__ kb, uint16_t* __restrict__ vb) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n_pairs;
       e += (int64_t)gridDim.x * blockDim.x) {
    ((uint32_t*)kb)[e] = pack_bf16x2(kbar[2 * e], kbar[2 * e + 1]);
    ((uint32_t*)vb)[e] = pack_bf16x2(vbar[2 * e], vbar[2 * e + 1]);
  }
}

// Split keys: coff[row][c] = first entry of the (ascending) kept list of row
// whose tile index is at least c * chunk_tiles, c = 0..n_chunks. Lower bound
// by bisection; any contents of sel give an index in [0, top_k].
__global__ __launch_bounds__(256) void chunk_offsets_kernel(const int32_t* __restrict__ sel,
                                                            int64_t rows, int32_t top_k,
                                                            int32_t n_chunks, int32_t chunk_tiles,
                                                            int32_t* __restrict__ coff) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= rows * (n_chunks + 1)) return;
  const int64_t row = e / (n_chunks + 1);
  const int ch = (int)(e - row * (n_chunks + 1));
  const int32_t* s = sel + row * top_k;
  const int64_t target = (int64_t)ch * chunk_tiles;
  int lo = 0, hi = top_k;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (s[mid] < target) lo = mid + 1;
    else hi = mid;
  }
  coff[e] = lo;
}

// Split keys: merge the chunk partials of each query in chunk order. 16 lanes
// per query, 4 channels each.
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ part_o,
                                                      const float2* __restrict__ part_ml,
                                                      int32_t n_chunks, int64_t nq, int64_t rows,
                                                      void* o, int64_t ost, int64_t osh,
                                                      int32_t o_f32, float* __restrict__ lse) {
  const int64_t r = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);  // (head, query)
  if (r >= rows) return;
  const int sub = threadIdx.x & 15;
  const float2* ml = part_ml + r * n_chunks;
  // loads go out kB chunks at a time (the sums still run in chunk order)
  constexpr int kB = 8;
  float ref = -INFINITY;  // over the chunks with columns (l > 0)
  int ch = 0;
  for (; ch + kB <= n_chunks; ch += kB) {
    float2 m[kB];
#pragma unroll
    for (int j = 0; j < kB; ++j) m[j] = ml[ch + j];
#pragma unroll
    for (int j = 0; j < kB; ++j)
      if (m[j].y > 0.f) ref = fmaxf(ref, m[j].x);
  }
  for (; ch < n_chunks; ++ch)
    if (ml[ch].y > 0.f) ref = fmaxf(ref, ml[ch].x);
  const float* po = part_o + r * n_chunks * kHeadDim + 4 * sub;
  float l = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  auto add = [&](float2 m, f32x4 x) {
    const float w = m.y > 0.f ? __builtin_amdgcn_exp2f(m.x - ref) : 0.f;
    l = __builtin_fmaf(m.y, w, l);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(x[i], w, acc[i]);
  };
  for (ch = 0; ch + kB <= n_chunks; ch += kB) {
    float2 m[kB];
    f32x4 x[kB];
#pragma unroll
    for (int j = 0; j < kB; ++j) {
      m[j] = ml[ch + j];
      x[j] = *(const f32x4*)(po + (int64_t)(ch + j) * kHeadDim);
    }
#pragma unroll
    for (int j = 0; j < kB; ++j) add(m[j], x[j]);
  }
  for (; ch < n_chunks; ++ch) add(ml[ch], *(const f32x4*)(po + (int64_t)ch * kHeadDim));
  const float inv = l > 0.f ? 1.0f / l : 0.f;  // l == 0 only without any column
  const int64_t h = r / nq, q = r - h * nq;
  if (lse != nullptr && sub == 0) lse[r] = ref + __builtin_log2f(l);
  if (o_f32) {
    float* op = (float*)o + h * osh + q * ost + 4 * sub;
    *(f32x4*)op = f32x4{acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
  } else {
    uint16_t* op = (uint16_t*)o + h * osh + q * ost + 4 * sub;
    *(u32x2*)op = u32x2{pack_bf16x2(acc[0] * inv, acc[1] * inv),
                        pack_bf16x2(acc[2] * inv, acc[3] * inv)};
  }
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Keys per chunk of the split-key decomposition: K and V of one chunk of one
// head take kChunkKeys * 256 bytes. Ranges of at least four long chunks use
// the long ones: with phased walks the items in flight share a window of the
// chunk, not the whole chunk, so fewer chunks save partials and per-item work
// (measured at 512 views: 65,536 keys 3% faster than 32,768 or 98,304).
constexpr int64_t kChunkKeys = 32768;
constexpr int64_t kChunkKeysLong = 65536;
// Partial outputs take at most this much workspace; longer ranges use fewer,
// larger chunks.
constexpr double kMaxPartialBytes = 64.0 * (1ull << 30);

struct SplitPlan {
  int32_t n_chunks = 1, chunk_tiles = 0;
  size_t coff = 0, part_o = 0, part_ml = 0;  // workspace bytes of each
};

// Split only where the K/V traffic bounds the stage: 128-query tiles fetch half
// the bytes per flop and run compute-bound, and there the partials cost more
// than the L2 reuse saves.
SplitPlan split_plan(int64_t nq, int64_t tk, int32_t heads, int32_t q_tile, int32_t k_tile,
                     int32_t top_k) {
  SplitPlan sp;
  if (top_k >= tk || q_tile > 64) return sp;
  int64_t ct = (tk * k_tile >= 4 * kChunkKeysLong ? kChunkKeysLong : kChunkKeys) / k_tile;
  const double per_chunk = (double)heads * nq * (kHeadDim + 2) * sizeof(float);
  // one partial slot per chunk, plus one for the landmark columns
  const int64_t max_chunks = (int64_t)(kMaxPartialBytes / per_chunk) - 1;
  if (max_chunks < 2 || tk < 2 * ct) return sp;
  int64_t nc = (tk + ct - 1) / ct;
  if (nc > max_chunks) {  // widen the chunks to a multiple of k_tile landmark rows
    ct = ((tk + max_chunks - 1) / max_chunks + k_tile - 1) / k_tile * k_tile;
    nc = (tk + ct - 1) / ct;
  }
  if (nc < 2) return sp;
  const int64_t tq = (nq + q_tile - 1) / q_tile;
  sp.n_chunks = (int32_t)nc;
  sp.chunk_tiles = (int32_t)ct;
  sp.coff = align256((size_t)heads * tq * (nc + 1) * sizeof(int32_t));
  sp.part_o = align256((size_t)heads * nq * (nc + 1) * kHeadDim * sizeof(float));
  sp.part_ml = align256((size_t)heads * nq * (nc + 1) * sizeof(float2));
  return sp;
}

// Workgroups of the key-half kernel the current device runs at once (its
// occupancy per CU times the CUs), or 0 if the runtime cannot say.
template <int QT>
int64_t kh_items_at_once() {
  static std::atomic<int> per_cu{-1};
  int nb = per_cu.load(std::memory_order_relaxed);
  if (nb < 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, tile_sparse_kh_kernel<QT, false>, QT * 2,
                                                     0) !=
        hipSuccess) {
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

template <int QT, int KT>
hipError_t launch_kernel(const SparseParams& p, const int32_t* sel, hipStream_t s) {
  // one workgroup per item (the item loop serves the rest when the grid is capped)
  const int64_t grid = std::min<int64_t>(p.n_items, (int64_t)1 << 24);
  // key-half kernel: 64-key tiles, 64 or 128 queries, 128-byte key rows
  if constexpr (KT == 64 && QT >= 64) {
    if (p.kst == kHeadDim) {
      SparseParams pk = p;
      // phase the kept-list walks of split-key launches (short walks over one
      // chunk, many rounds of items); measured slower on whole key ranges
      const int64_t period = p.n_chunks > 1 ? kh_items_at_once<QT>() : 0;
      pk.phase_period = sel != nullptr && period > 0 && p.n_items >= 4 * period ? period : 0;
      hipLaunchKernelGGL((tile_sparse_kh_kernel<QT, false>), dim3((unsigned)grid), dim3(QT * 2), 0, s,
                         pk, sel);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((tile_sparse_kernel<QT, KT>), dim3((unsigned)grid), dim3(QT * 2), 0, s, p,
                     sel);
  return hipGetLastError();
}

hipError_t launch_tiles(const SparseParams& p, const int32_t* sel, int32_t q_tile,
                        int32_t k_tile, hipStream_t s) {
  if (k_tile == 64) {
    if (q_tile == 32) return launch_kernel<32, 64>(p, sel, s);
    if (q_tile == 64) return launch_kernel<64, 64>(p, sel, s);
    return launch_kernel<128, 64>(p, sel, s);
  }
  if (q_tile == 32) return launch_kernel<32, 32>(p, sel, s);
  if (q_tile == 64) return launch_kernel<64, 32>(p, sel, s);
  return launch_kernel<128, 32>(p, sel, s);
}

}  // namespace

size_t sparse_workspace_bytes(int64_t n_q, int64_t n_kv, int32_t heads, int32_t q_tile,
                              int32_t k_tile, int32_t top_k) {
  const int64_t tk = (n_kv + k_tile - 1) / k_tile;
  const size_t range = align256((size_t)heads * kRangeParts * 2 * sizeof(float));
  if (top_k >= tk) return range;
  const size_t lm = align256((size_t)heads * tk * kHeadDim * sizeof(uint16_t));
  const SplitPlan sp = split_plan(n_q, tk, heads, q_tile, k_tile, top_k);
  return 2 * lm + range + sp.coff + sp.part_o + sp.part_ml;
}

hipError_t launch_pack_landmarks(const float* kbar, const float* vbar, int32_t heads, int32_t tk,
                                 uint16_t* kb, uint16_t* vb, hipStream_t s) {
  const int64_t pairs = (int64_t)heads * tk * (kHeadDim / 2);
  if (pairs == 0) return hipSuccess;
  const int blocks = (int)std::min<int64_t>((pairs + 255) / 256, 8192);
  hipLaunchKernelGGL(pack_landmarks_kernel, dim3(blocks), dim3(256), 0, s, kbar, vbar, pairs, kb,
                     vb);
  return hipGetLastError();
}

hipError_t launch_tile_sparse(const uint16_t* q, int64_t nq, int64_t qst, int64_t qsh,
                              const uint16_t* k, const uint16_t* v, int64_t nk, int64_t kst,
                              int64_t ksh, int32_t heads, const float* kbar, const float* vbar,
                              const int32_t* sel, int32_t q_tile, int32_t k_tile,
                              int32_t top_k, float scale, void* o, int64_t ost, int64_t osh,
                              bool o_f32, uint32_t flags, void* ws, hipStream_t s,
                              float* lse) {
  SparseParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.nq = nq;
  p.qst = qst;
  p.qsh = qsh;
  p.nk = nk;
  p.kst = kst;
  p.ksh = ksh;
  p.ost = ost;
  p.osh = osh;
  p.tq = (int32_t)((nq + q_tile - 1) / q_tile);
  p.tk = (int32_t)((nk + k_tile - 1) / k_tile);
  p.n_items = (int64_t)heads * p.tq;
  p.n_chunks = 1;
  p.chunk_tiles = 0;
  p.coff = nullptr;
  p.part_o = nullptr;
  p.part_ml = nullptr;
  p.lse = lse;
  p.phase_period = 0;
  p.part_slots = 1;
  p.lm_separate = 0;
  p.tq_sel = p.tq;
  p.top_k = top_k;
  p.scale_log2 = scale * kLog2e;
  p.o_f32 = o_f32 ? 1 : 0;
  p.kbar_b = nullptr;
  p.vbar_b = nullptr;
  p.landmarks = (flags & kSparseNoLandmarks) ? 0 : 1;
  p.log_count = (flags & kSparseLandmarkLogCount) ? 1 : 0;
  p.lm_log2_kt = __builtin_log2f((float)k_tile);
  {
    const int64_t tail = nk - (int64_t)(p.tk - 1) * k_tile;  // tokens of the last key tile
    p.lm_tail_corr = tail > 0 ? (__builtin_log2f((float)tail) - p.lm_log2_kt) / (scale * kLog2e)
                              : 0.f;
  }
  if (p.tq == 0 || heads == 0) return hipSuccess;
  const bool sparse = sel != nullptr && top_k < p.tk;
  uint8_t* wsb = (uint8_t*)ws;
  if (sparse) {
    const size_t lm = align256((size_t)heads * p.tk * kHeadDim * sizeof(uint16_t));
    wsb += 2 * lm;
  }
  if (sparse && p.landmarks) {
    const size_t lm = align256((size_t)heads * p.tk * kHeadDim * sizeof(uint16_t));
    uint16_t* kb = (uint16_t*)ws;
    uint16_t* vb = (uint16_t*)((uint8_t*)ws + lm);
    hipError_t err = launch_pack_landmarks(kbar, vbar, heads, p.tk, kb, vb, s);
    if (err != hipSuccess) return err;
    p.kbar_b = kb;
    p.vbar_b = vb;
  }
  if (!sparse) sel = nullptr;  // every tile kept: dense attention, no landmarks
  float* range = (float*)wsb;
  hipLaunchKernelGGL(range_kernel, dim3(kRangeParts, heads), dim3(256), 0, s, k, v, nk, kst, ksh,
                     p.kbar_b, p.vbar_b, p.tk, range);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  p.range = range;
  const SplitPlan sp = sparse ? split_plan(nq, p.tk, heads, q_tile, k_tile, top_k) : SplitPlan{};
  if (sp.n_chunks == 1) return launch_tiles(p, sel, q_tile, k_tile, s);

  uint8_t* w = wsb + align256((size_t)heads * kRangeParts * 2 * sizeof(float));
  p.n_chunks = sp.n_chunks;
  p.chunk_tiles = sp.chunk_tiles;
  p.coff = (const int32_t*)w;
  p.part_o = (float*)(w + sp.coff);
  p.part_ml = (float2*)(w + sp.coff + sp.part_o);
  p.n_items = (int64_t)heads * sp.n_chunks * p.tq;
  // the key-half kernel's 64-query items leave their landmark blocks to one
  // pass of 128-query items (pairs of query tiles) over all landmark rows, which
  // halves the landmark blocks' gathers; that pass, run last, also merges the
  // chunks' partials (its own partial is the last slot, kept in registers)
  const bool lm_pass = p.landmarks && q_tile == 64 && k_tile == 64 && kst == kHeadDim;
  p.lm_separate = lm_pass ? 1 : 0;
  p.part_slots = sp.n_chunks + (lm_pass ? 1 : 0);
  const int64_t rows = (int64_t)heads * p.tq;
  const int64_t n_off = rows * (sp.n_chunks + 1);
  hipLaunchKernelGGL(chunk_offsets_kernel, dim3((unsigned)((n_off + 255) / 256)), dim3(256), 0, s,
                     sel, rows, top_k, sp.n_chunks, sp.chunk_tiles, (int32_t*)w);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if ((err = launch_tiles(p, sel, q_tile, k_tile, s)) != hipSuccess) return err;
  if (lm_pass) {
    SparseParams pl = p;
    pl.tq_sel = p.tq;
    pl.tq = (p.tq + 1) / 2;  // pairs of 64-query tiles
    pl.n_items = (int64_t)heads * pl.tq;
    pl.phase_period = 0;
    hipLaunchKernelGGL((tile_sparse_kh_kernel<128, true>),
                       dim3((unsigned)std::min<int64_t>(pl.n_items, (int64_t)1 << 24)), dim3(256),
                       0, s, pl, sel);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (lm_pass) return hipSuccess;  // the landmark pass merged the partials
  const int64_t qrows = (int64_t)heads * nq;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((qrows + 15) / 16)), dim3(256), 0, s,
                     (const float*)p.part_o, (const float2*)p.part_ml, p.part_slots, nq, qrows,
                     o, ost, osh, p.o_f32, lse);
  return hipGetLastError();
}

}  // namespace zebra
