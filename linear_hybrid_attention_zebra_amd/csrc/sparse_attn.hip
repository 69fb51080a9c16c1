// Tile-sparse softmax attention with mean-key/value landmarks (gfx950).
//
// Zebra3D paper page (thelatestinai.com), Figure 1 caption: kept tiles keep
// full softmax interactions; omitted tiles become mean-key/value landmarks.
// For every query of query tile i the softmax runs over every token of the
// kept key tiles sel[h][i][*] plus one landmark column (kbar_j, vbar_j) for
// each omitted tile j. With sel == NULL every tile is kept: exact dense
// attention.
//
// One workgroup per (head, query tile), one wave per 32 queries. Each query
// tile walks one list of column blocks: its kept key tiles (ascending), then
// its omitted tiles' landmarks, KT at a time. For each block the wave
// computes the transposed score block S^T = K Q^T with bf16 MFMA 32x32x16, so
// that each lane holds the scores of ONE query over 32 keys; the online
// softmax (base-2, float32) is then lane-local except for one exchange with
// the lane 32 apart (v_permlane32_swap). The probabilities, rounded to bf16,
// are already in the B-operand layout of the second MFMA O^T += V^T P^T; V
// stays row-major in LDS and is read transposed with ds_read_b64_tr_b16.
// Rescaling of O and l is lazy: the running maximum moves only when a block's
// maximum exceeds it by more than 8 (log2 units), so every probability is
// <= 2^8. The row sum is accumulated from the bf16-rounded probabilities
// (v_dot2 with ones), the same values the PV product uses.
//
// Blocks go global -> LDS directly (global_load_lds_dwordx4) into a ring of
// STAGES buffers, later blocks' loads in flight while the current block
// computes; one barrier per block. 16-byte LDS chunks are XOR swizzled by row
// so the MFMA operand reads spread over the banks. The block list is read
// from a small LDS window, refilled every kWin entries.
#include <algorithm>
#include <type_traits>

#include "common.h"

namespace zebra {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleSlack = 8.0f;
constexpr int kWin = 2048;  // entries of the block-list window in LDS

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;  // LDS bytes

struct SparseParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* kbar_b;  // bf16 landmarks [H][tk][64]
  const uint16_t* vbar_b;
  const uint16_t* omit;    // [H][tq][tk - top_k] omitted tiles, ascending
  void* o;
  int64_t nq, qst, qsh;
  int64_t nk, kst, ksh;
  int64_t ost, osh;
  int32_t tq, tk, top_k;
  float scale_log2;  // softmax scale * log2(e)
  int32_t o_f32;
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
// loads of blocks still in flight. LDS reads are complete (lgkmcnt) first; the
// loads of the block about to be read are waited for explicitly (vmcnt).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0f70 | (N & 15) | ((N >> 4) << 14));
}

template <int QT, int KT, int STAGES>
__global__ __launch_bounds__(QT * 2) void tile_sparse_kernel(SparseParams p,
                                                             const int32_t* __restrict__ sel) {
  constexpr int W = QT / 32;             // waves
  constexpr int NT = W * kWave;          // threads
  constexpr int NB = KT / 32;            // 32-key score blocks per tile
  constexpr int TILE_BYTES = KT * 128;   // one K (or V) block in LDS
  constexpr int KB_PER_TILE = TILE_BYTES / 1024;  // 1 KB direct-to-LDS wave loads
  constexpr int NU = KB_PER_TILE / W;    // 1 KB blocks per wave per tensor
  constexpr int LOADS_PER_TILE = 2 * NU; // this wave's DMA instructions per block
  static_assert(KB_PER_TILE % W == 0, "load split");
  static_assert(STAGES >= 2 && STAGES <= 3 && (STAGES - 2) * LOADS_PER_TILE <= 63,
                "ring depth");

  // One K and one V array per ring stage. Distinct LDS objects, indexed with
  // compile-time stage numbers, let the compiler prove that reads of one stage
  // do not alias the direct-to-LDS writes still in flight to another, so it
  // does not wait for those loads before every LDS read.
  // [1 KB block][16-byte chunk of lane] of each K and V stage
  __shared__ u32x4 ks0[KB_PER_TILE][64], vs0[KB_PER_TILE][64];
  __shared__ u32x4 ks1[KB_PER_TILE][64], vs1[KB_PER_TILE][64];
  __shared__ u32x4 ks2[STAGES > 2 ? KB_PER_TILE : 1][64], vs2[STAGES > 2 ? KB_PER_TILE : 1][64];
  __shared__ uint16_t win[kWin];
  typedef __attribute__((address_space(3))) u32x4 lds_blk[64];
  auto kbuf = [&](auto stc) -> lds_blk* {
    constexpr int S = decltype(stc)::value;
    if constexpr (S == 0) return (lds_blk*)ks0;
    else if constexpr (S == 1) return (lds_blk*)ks1;
    else return (lds_blk*)ks2;
  };
  auto vbuf = [&](auto stc) -> lds_blk* {
    constexpr int S = decltype(stc)::value;
    if constexpr (S == 0) return (lds_blk*)vs0;
    else if constexpr (S == 1) return (lds_blk*)vs1;
    else return (lds_blk*)vs2;
  };

  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int qi = lane & 31;   // query within the wave / column of S^T
  const int hh = lane >> 5;   // lane half
  const int h = blockIdx.x / p.tq;
  const int qtile = blockIdx.x % p.tq;
  const bool dense = sel == nullptr;
  const int n_kept = dense ? p.tk : p.top_k;
  const int n_omit = dense ? 0 : p.tk - p.top_k;
  const int n_lblk = (n_omit + KT - 1) / KT;
  const int n_total = n_kept + n_lblk;
  const int n_list = n_kept + n_omit;  // entries of the block list
  const int32_t* sel_row = dense ? nullptr : sel + ((int64_t)h * p.tq + qtile) * p.top_k;
  const uint16_t* omit_row =
      n_omit > 0 ? p.omit + ((int64_t)h * p.tq + qtile) * n_omit : nullptr;

  // ---- query operand (B of S^T = K Q^T): Q[q][16s + 8hh .. +7]
  const int64_t qrow = (int64_t)qtile * QT + wave * 32 + qi;
  const bool qvalid = qrow < p.nq;
  bf16x8 qop[4];
  {
    const uint16_t* qp = p.q + (int64_t)h * p.qsh + qrow * p.qst + 8 * hh;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (qvalid) w = *(const u32x4*)(qp + 16 * s);
      qop[s] = as_bf16x8(w);
    }
  }

  // the only short key tile is the last one, kept last when kept at all
  const int last_kept = dense ? p.tk - 1 : min(max(sel_row[n_kept - 1], 0), p.tk - 1);
  // Complete these vector loads now, before any direct-to-LDS load is issued:
  // afterwards the vector-memory counter also counts the ring's loads, and a
  // late first use of qop would otherwise wait for all of them.
  wait_vmcnt<0>();
  const int tail_rows = (int)(p.nk - (int64_t)(p.tk - 1) * KT);  // rows of tile tk-1
  const int last_rows = last_kept == p.tk - 1 ? tail_rows : KT;
  const int last_lrows = n_omit - (n_lblk - 1) * KT;  // columns of the last landmark block

  // ---- block-list window: entries [win_lo, win_lo + kWin) of
  // (kept tiles..., omitted tiles...). Refilled by all threads together.
  int win_lo = 0;
  auto refill = [&](int lo) {
    win_lo = lo;
    for (int e = tid; e < kWin; e += NT) {
      const int pos = lo + e;
      int j = 0;
      if (pos < n_kept)
        j = sel_row[pos];
      else if (pos < n_list)
        j = omit_row[pos - n_kept];
      win[e] = (uint16_t)min(max(j, 0), p.tk - 1);
    }
    __syncthreads();
  };

  f32x16 oacc[2];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    oacc[0][i] = 0.f;
    oacc[1][i] = 0.f;
  }
  const float c = p.scale_log2;  // raw score -> log2 units
  float mc_run = -INFINITY;      // running max in log2 units
  float l_run = 0.f;
  const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3f803f80u);

  // ---- direct-to-LDS staging. 1 KB block u of a tile holds rows 8u..8u+7;
  // lane i writes physical chunk i%8 of row r = 8u + i/8, i.e. logical chunk
  // (i%8) ^ swz_f(r). This wave stages blocks u = wave + W v.
  const int lrow = lane >> 3;
  int lchunk[NU];
  uint32_t off_kv[NU];
#pragma unroll
  for (int v = 0; v < NU; ++v) {
    const int r = 8 * (wave + W * v) + lrow;
    lchunk[v] = (lane & 7) ^ swz_f(r);
    off_kv[v] = (uint32_t)(r * p.kst * 2 + lchunk[v] * 16);
  }
  auto dma = [&](const void* src, lds_blk* dst, int u) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)&dst[u][0], 16,
                                     0, 0);
  };
  const uint8_t* kh = (const uint8_t*)(p.k + (int64_t)h * p.ksh);
  const uint8_t* vh = (const uint8_t*)(p.v + (int64_t)h * p.ksh);
  const uint8_t* klm = dense ? nullptr : (const uint8_t*)(p.kbar_b + (int64_t)h * p.tk * kHeadDim);
  const uint8_t* vlm = dense ? nullptr : (const uint8_t*)(p.vbar_b + (int64_t)h * p.tk * kHeadDim);

  auto issue = [&](int t, auto stc) {  // stage block t of the list into stage stc
    // per-lane source offsets for the three kinds of block, then one set of
    // loads: a full kept tile, the short last tile (rows clamped to its last
    // valid row), or landmark rows gathered by index (rows past the list
    // repeat its last entry)
    const uint8_t* kb;
    const uint8_t* vb;
    uint32_t off[NU];
    if (t < n_kept) {
      const int j = dense ? t : win[t - win_lo];
      const int64_t base = (int64_t)j * KT * p.kst * 2;
      kb = kh + base;
      vb = vh + base;
      const bool short_tile = j == p.tk - 1 && tail_rows < KT;
#pragma unroll
      for (int v = 0; v < NU; ++v) {
        const int r = min(8 * (wave + W * v) + lrow, tail_rows - 1);
        off[v] = short_tile ? (uint32_t)(r * p.kst * 2 + lchunk[v] * 16) : off_kv[v];
      }
    } else {
      const int e0 = n_kept + (t - n_kept) * KT - win_lo;
      const int rows = t == n_total - 1 ? last_lrows : KT;
      kb = klm;
      vb = vlm;
#pragma unroll
      for (int v = 0; v < NU; ++v) {
        const int r = min(8 * (wave + W * v) + lrow, rows - 1);
        off[v] = (uint32_t)win[e0 + r] * 128u + (uint32_t)lchunk[v] * 16u;
      }
    }
    lds_blk* kd = kbuf(stc);
    lds_blk* vd = vbuf(stc);
#pragma unroll
    for (int v = 0; v < NU; ++v) {
      dma(kb + off[v], kd, wave + W * v);
      dma(vb + off[v], vd, wave + W * v);
    }
  };
  // list entries block t reads: [first, first + count)
  auto ensure_window = [&](int t) {  // collective; t is uniform
    if (dense) return;
    int first, count;
    if (t < n_kept) {
      first = t;
      count = 1;
    } else {
      first = n_kept + (t - n_kept) * KT;
      count = min(KT, n_list - first);
    }
    if (first < win_lo || first + count > win_lo + kWin) {
      lds_barrier();  // earlier issues (all waves) have read the old window
      refill(first);
    }
  };

  // ---- one block of KT columns from stage `st`; `colmask` bit set = column
  // excluded (looked at only when the tag says so)
  auto compute_tile = [&](auto stc, auto masked_tag, uint64_t colmask) {
    constexpr bool kMasked = decltype(masked_tag)::value;
    const lds_u8* ks = (const lds_u8*)kbuf(stc);
    const lds_u8* vs = (const lds_u8*)vbuf(stc);
    f32x16 sacc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[b][i] = 0.f;
      const int row = 32 * b + qi;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8 a =
            as_bf16x8(*(const __attribute__((address_space(3))) u32x4*)(ks + swz(row, 2 * s + hh)));
        sacc[b] = mfma32(a, qop[s], sacc[b]);
      }
    }
    // lane holds keys 32b + 8g + 4hh + r in register 4g + r of block b
    if constexpr (kMasked) {
      const uint64_t cm = colmask >> (4 * hh);
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int bit = 32 * b + 8 * (i >> 2) + (i & 3);
          if ((cm >> bit) & 1ull) sacc[b][i] = -INFINITY;
        }
    }
    // block maximum: two independent v_maximum3 chains (NaN-propagating
    // maximum needs no operand canonicalisation, unlike fmaxf)
    float tm0 = sacc[0][0], tm1 = sacc[0][1];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = (b == 0 ? 2 : 0); i < 16; i += 2) {
        tm0 = __builtin_elementwise_maximum(tm0, sacc[b][i]);
        tm1 = __builtin_elementwise_maximum(tm1, sacc[b][i + 1]);
      }
    float tmax = __builtin_elementwise_maximum(tm0, tm1);
    {
      // v_permlane32_swap with both operands = tmax: lanes 0-31 receive the
      // partner value in the second result, lanes 32-63 in the first; the
      // other result is the lane's own value, so max(r0, r1) is the row max.
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax),
                                                       __float_as_uint(tmax), false, false);
      tmax = __builtin_elementwise_maximum(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    const float tmc = tmax * c;
    if (__any(tmc > mc_run + kRescaleSlack)) {
      const float m_new = __builtin_elementwise_maximum(mc_run, tmc);
      const float alpha = __builtin_amdgcn_exp2f(mc_run - m_new);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        oacc[0][i] *= alpha;
        oacc[1][i] *= alpha;
      }
      l_run *= alpha;
      mc_run = m_new;
    }
    const float nmc = -mc_run;
    bf16x8 pop[2 * NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      uint32_t w[8];
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[b][i], c, nmc));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[b][i + 1], c, nmc));
        w[i >> 1] = pack_bf16x2(p0, p1);
        l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[i >> 1]), ones,
                                                l_run, false);
      }
      u32x4 lo = {w[0], w[1], w[2], w[3]}, hi = {w[4], w[5], w[6], w[7]};
      pop[2 * b] = as_bf16x8(lo);
      pop[2 * b + 1] = as_bf16x8(hi);
    }
    // O^T[d][q] += V^T[d][key] P^T[key][q], 16 keys per MFMA. Lane group
    // G = lane/16 covers d offset 16(G%2) and key half G/2; each of the two
    // transposed reads returns 4 consecutive keys for the lane's channel.
    const int G = lane >> 4, S = lane & 15;
#pragma unroll
    for (int m = 0; m < KT / 16; ++m) {
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        const int col = 32 * db + 16 * (G & 1) + 4 * (S & 3);
        const int chunk = col >> 3, half = (col & 7) ? 8 : 0;
        const int r0 = 16 * m + 4 * (G >> 1) + (S >> 2);
        const int r1 = r0 + 8;
        const i16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(vs + swz(r0, chunk) + half));
        const i16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(vs + swz(r1, chunk) + half));
        const u32x2 w0 = __builtin_bit_cast(u32x2, t0), w1 = __builtin_bit_cast(u32x2, t1);
        const u32x4 w = {w0.x, w0.y, w1.x, w1.y};
        oacc[db] = mfma32(as_bf16x8(w), pop[m], oacc[db]);
      }
    }
  };

  // ---- the block sequence through a ring of STAGES buffers: block t lives in
  // stage t % STAGES; loads of blocks t+1 .. t+STAGES-2 may be in flight
  // while block t computes. The loop is unrolled by STAGES so that every
  // stage index is a compile-time constant.
  // Every step issues exactly one block's loads (past the end of the list it
  // re-loads the last block into the stage that is free) and waits for the
  // same count. The first STAGES-1 steps (t < 0) only issue: they are the
  // prologue, folded into the loop so that the loop is entered with no load
  // in flight. With one uniform load stream the compiler's view of the
  // outstanding loads is exact and it adds no waits of its own.
  if (!dense) refill(0);
  auto step = [&](int t, auto stc) {
    constexpr int ST = decltype(stc)::value;  // stage of block t
    constexpr int NEXT = (ST + STAGES - 1) % STAGES;
    // this wave's loads of block t have landed once no more than the loads of
    // the (STAGES - 2) later blocks already issued remain outstanding
    wait_vmcnt<(STAGES - 2) * LOADS_PER_TILE>();
    lds_barrier();  // every wave's loads of block t landed; stage NEXT is free
    const int tn = min(t + STAGES - 1, n_total - 1);
    ensure_window(tn);
    issue(tn, std::integral_constant<int, NEXT>{});
    if (t < 0) return;
    if (t < n_kept) {
      if (t == n_kept - 1 && last_rows < KT)
        compute_tile(stc, std::true_type{}, ~0ull << last_rows);
      else
        compute_tile(stc, std::false_type{}, 0ull);
    } else {
      if (t == n_total - 1 && last_lrows < KT)
        compute_tile(stc, std::true_type{}, ~0ull << last_lrows);
      else
        compute_tile(stc, std::false_type{}, 0ull);
    }
  };
  // rounds of STAGES unconditional steps; position p of a round holds a block
  // of stage (p + 1) % STAGES because the first round starts at t = 1 - STAGES
  using S0 = std::integral_constant<int, 1 % STAGES>;
  using S1 = std::integral_constant<int, 2 % STAGES>;
  using S2 = std::integral_constant<int, 3 % STAGES>;
  int t = 1 - STAGES;
  for (; t + STAGES <= n_total; t += STAGES) {
    step(t, S0{});
    step(t + 1, S1{});
    if constexpr (STAGES > 2) step(t + 2, S2{});
  }
  if (t < n_total) step(t, S0{});
  if constexpr (STAGES > 2) {
    if (t + 1 < n_total) step(t + 1, S1{});
  }
  wait_vmcnt<0>();  // no direct-to-LDS load may outlive the workgroup's LDS

  // ---- epilogue: O / l, lane (qi, hh) holds channels 32db + 8g + 4hh + r
  const auto lsw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run),
                                                    __float_as_uint(l_run), false, false);
  const float inv = 1.0f / (__uint_as_float(lsw[0]) + __uint_as_float(lsw[1]));  // own + partner
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

// Omitted tiles of every (head, query tile): the complement of its ascending
// kept list, ascending. Gap g lies between kept tiles g-1 and g; omitted tile
// j in gap g sits at position j - g.
__global__ __launch_bounds__(256) void complement_kernel(const int32_t* __restrict__ sel,
                                                         int32_t top_k, int32_t tk,
                                                         uint16_t* __restrict__ omit) {
  const int64_t row = blockIdx.x;
  const int32_t* s = sel + row * top_k;
  uint16_t* out = omit + row * (int64_t)(tk - top_k);
  for (int g = threadIdx.x; g <= top_k; g += 256) {
    const int lo = g == 0 ? 0 : min(max(s[g - 1], -1), tk - 1) + 1;
    const int hi = g == top_k ? tk : min(max(s[g], 0), tk);
    for (int j = lo; j < hi; ++j) {
      const int pos = j - g;
      if (pos >= 0 && pos < tk - top_k) out[pos] = (uint16_t)j;
    }
  }
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

template <int QT, int KT, int STAGES>
hipError_t launch_kernel(const SparseParams& p, const int32_t* sel, int heads, hipStream_t s) {
  const int64_t blocks = (int64_t)heads * p.tq;
  hipLaunchKernelGGL((tile_sparse_kernel<QT, KT, STAGES>), dim3((unsigned)blocks), dim3(QT * 2),
                     0, s, p, sel);
  return hipGetLastError();
}

}  // namespace

size_t sparse_workspace_bytes(int64_t n_q, int64_t n_kv, int32_t heads, int32_t q_tile,
                              int32_t k_tile, int32_t top_k) {
  const int64_t tk = (n_kv + k_tile - 1) / k_tile;
  const int64_t tq = (n_q + q_tile - 1) / q_tile;
  if (top_k >= tk) return 0;
  const size_t lm = align256((size_t)heads * tk * kHeadDim * sizeof(uint16_t));
  return 2 * lm + align256((size_t)heads * tq * (tk - top_k) * sizeof(uint16_t));
}

hipError_t launch_tile_sparse(const uint16_t* q, int64_t nq, int64_t qst, int64_t qsh,
                              const uint16_t* k, const uint16_t* v, int64_t nk, int64_t kst,
                              int64_t ksh, int32_t heads, const float* kbar, const float* vbar,
                              const int32_t* sel, int32_t q_tile, int32_t k_tile,
                              int32_t top_k, float scale, void* o, int64_t ost, int64_t osh,
                              bool o_f32, void* ws, hipStream_t s) {
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
  p.top_k = top_k;
  p.scale_log2 = scale * kLog2e;
  p.o_f32 = o_f32 ? 1 : 0;
  p.kbar_b = nullptr;
  p.vbar_b = nullptr;
  p.omit = nullptr;
  if (p.tq == 0 || heads == 0) return hipSuccess;
  if (sel != nullptr && top_k < p.tk) {
    const size_t lm = align256((size_t)heads * p.tk * kHeadDim * sizeof(uint16_t));
    uint16_t* kb = (uint16_t*)ws;
    uint16_t* vb = (uint16_t*)((uint8_t*)ws + lm);
    uint16_t* om = (uint16_t*)((uint8_t*)ws + 2 * lm);
    const int64_t pairs = (int64_t)heads * p.tk * (kHeadDim / 2);
    const int blocks = (int)std::min<int64_t>((pairs + 255) / 256, 8192);
    hipLaunchKernelGGL(pack_landmarks_kernel, dim3(blocks), dim3(256), 0, s, kbar, vbar, pairs,
                       kb, vb);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(complement_kernel, dim3((unsigned)((int64_t)heads * p.tq)), dim3(256), 0,
                       s, sel, top_k, p.tk, om);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    p.kbar_b = kb;
    p.vbar_b = vb;
    p.omit = om;
  } else {
    sel = nullptr;  // every tile kept: dense attention, no landmarks
  }
  if (k_tile == 64) {
    if (q_tile == 32) return launch_kernel<32, 64, 2>(p, sel, heads, s);
    if (q_tile == 64) return launch_kernel<64, 64, 2>(p, sel, heads, s);
    return launch_kernel<128, 64, 2>(p, sel, heads, s);
  }
  if (q_tile == 32) return launch_kernel<32, 32, 3>(p, sel, heads, s);
  if (q_tile == 64) return launch_kernel<64, 32, 3>(p, sel, heads, s);
  return launch_kernel<128, 32, 3>(p, sel, heads, s);
}

}  // namespace zebra
