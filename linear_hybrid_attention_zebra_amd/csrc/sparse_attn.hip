// Tile-sparse softmax attention with mean-key/value landmarks (gfx950).
//
// Zebra3D paper page (thelatestinai.com), Figure 1 caption: kept tiles keep
// full softmax interactions; omitted tiles become mean-key/value landmarks.
// For every query of query tile i the softmax runs over every token of the
// kept key tiles sel[h][i][*] plus one landmark column (kbar_j, vbar_j) for
// each omitted tile j. With sel == NULL every tile is kept: exact dense
// attention.
//
// One workgroup per (head, query tile), one wave per 32 queries. For each
// kept key tile (ascending) and then each block of landmarks, the wave
// computes the transposed score block S^T = K Q^T with bf16 MFMA 32x32x16, so
// that each lane holds the scores of ONE query over 32 keys; the online
// softmax (base-2, float32) is then lane-local except for one exchange with
// the lane 32 apart. The probabilities, rounded to bf16, are already in the
// B-operand layout of the second MFMA O^T += V^T P^T; V stays row-major in
// LDS and is read transposed with ds_read_b64_tr_b16. Rescaling of O and l
// is lazy: the running maximum moves only when a tile's maximum exceeds it by
// more than 8 (in log2 units), which keeps every probability <= 2^8.
//
// K and V tiles are staged global -> registers -> LDS, the next tile's loads
// in flight while the current tile computes. 16-byte LDS chunks are XOR
// swizzled by (row & 7) so the MFMA operand reads are bank-conflict free.
#include <algorithm>
#include <type_traits>

#include "common.h"

namespace zebra {

namespace {

constexpr int kMaxTk = 32768;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleSlack = 8.0f;

typedef short i16x4 __attribute__((ext_vector_type(4)));

struct SparseParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* kbar_b;  // bf16 landmarks [H][tkp][64], zero rows past tk
  const uint16_t* vbar_b;
  const int32_t* sel;      // [H][tq][top_k] or nullptr (dense)
  void* o;
  int64_t nq, qst, qsh;
  int64_t nk, kst, ksh;
  int64_t ost, osh;
  int32_t tq, tk, tkp, top_k;
  float scale_log2;  // softmax scale * log2(e)
  int32_t o_f32;
};

__device__ __forceinline__ uint32_t swz(int row, int chunk) {
  return (uint32_t)(row * 128 + ((chunk ^ (row & 7)) << 4));
}

template <int QT, int KT>
__global__ __launch_bounds__(QT * 2) void tile_sparse_kernel(SparseParams p) {
  constexpr int W = QT / 32;         // waves
  constexpr int NT = W * kWave;      // threads
  constexpr int CPT = KT * 8 / NT;   // 16-byte chunks per thread per tensor
  constexpr int NB = KT / 32;        // 32-key score blocks per tile
  static_assert(CPT >= 1 && KT * 8 % NT == 0, "tile/threads mismatch");

  __shared__ __attribute__((aligned(16))) uint8_t ks[KT * 128];
  __shared__ __attribute__((aligned(16))) uint8_t vs[KT * 128];
  __shared__ uint32_t bitmap[kMaxTk / 32];

  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int qi = lane & 31;   // query within the wave / column of S^T
  const int hh = lane >> 5;   // lane half
  const int h = blockIdx.x / p.tq;
  const int qtile = blockIdx.x % p.tq;
  const bool dense = p.sel == nullptr;
  const int32_t* sel_row = dense ? nullptr : p.sel + ((int64_t)h * p.tq + qtile) * p.top_k;

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

  // ---- omitted-tile bitmap (bit j set = tile j kept)
  if (!dense) {
    const int words = (p.tk + 31) / 32;
    for (int w = tid; w < words; w += NT) bitmap[w] = 0u;
    __syncthreads();
    for (int t = tid; t < p.top_k; t += NT) {
      const int j = sel_row[t];
      if (j >= 0 && j < p.tk) atomicOr(&bitmap[j >> 5], 1u << (j & 31));
    }
    __syncthreads();
  }

  f32x16 oacc[2];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    oacc[0][i] = 0.f;
    oacc[1][i] = 0.f;
  }
  float m_run = -INFINITY;
  float l_run = 0.f;

  // ---- staging: rows r of the current tile, chunk c; invalid rows are zero
  u32x4 kreg[CPT], vreg[CPT];
  auto load_tile = [&](const uint16_t* kb, const uint16_t* vb, int64_t rstride, int nrows) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int e = tid + NT * u;
      const int r = e >> 3, c = e & 7;
      u32x4 kw = {0u, 0u, 0u, 0u}, vw = {0u, 0u, 0u, 0u};
      if (r < nrows) {
        kw = *(const u32x4*)(kb + r * rstride + 8 * c);
        vw = *(const u32x4*)(vb + r * rstride + 8 * c);
      }
      kreg[u] = kw;
      vreg[u] = vw;
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int e = tid + NT * u;
      const int r = e >> 3, c = e & 7;
      *(u32x4*)(ks + swz(r, c)) = kreg[u];
      *(u32x4*)(vs + swz(r, c)) = vreg[u];
    }
  };

  // ---- one tile of KT columns; `colmask` bit set = column excluded (only
  // looked at when the tag says the tile has excluded columns)
  auto compute_tile = [&](auto masked_tag, uint64_t colmask) {
    constexpr bool kMasked = decltype(masked_tag)::value;
    f32x16 sacc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[b][i] = 0.f;
      const int row = 32 * b + qi;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8 a = as_bf16x8(*(const u32x4*)(ks + swz(row, 2 * s + hh)));
        sacc[b] = mfma32(a, qop[s], sacc[b]);
      }
    }
    // scores -> log2 domain, masked columns -> -inf; lane holds keys
    // 32b + 8g + 4hh + r in register 4g + r of block b
    float tmax = -INFINITY;
    const uint64_t cm = colmask >> (4 * hh);
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float x = sacc[b][i] * p.scale_log2;
        if constexpr (kMasked) {
          const int bit = 32 * b + 8 * (i >> 2) + (i & 3);
          if ((cm >> bit) & 1ull) x = -INFINITY;
        }
        sacc[b][i] = x;
        tmax = fmaxf(tmax, x);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
    if (__any(tmax > m_run + kRescaleSlack)) {
      const float m_new = fmaxf(m_run, tmax);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        oacc[0][i] *= alpha;
        oacc[1][i] *= alpha;
      }
      l_run *= alpha;
      m_run = m_new;
    }
    bf16x8 pop[2 * NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      uint32_t w[8];
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const float p0 = __builtin_amdgcn_exp2f(sacc[b][i] - m_run);
        const float p1 = __builtin_amdgcn_exp2f(sacc[b][i + 1] - m_run);
        l_run += p0 + p1;
        w[i >> 1] = pack_bf16x2(p0, p1);
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

  // ---- phase 1: kept tiles (ascending), or every tile when dense
  const int n_kept = dense ? p.tk : p.top_k;
  const uint16_t* kh = p.k + (int64_t)h * p.ksh;
  const uint16_t* vh = p.v + (int64_t)h * p.ksh;
  auto tile_of = [&](int t) {
    int j = dense ? t : sel_row[t];
    return min(max(j, 0), p.tk - 1);
  };
  auto tile_rows = [&](int j) { return (int)min((int64_t)KT, p.nk - (int64_t)j * KT); };
  {
    int j = tile_of(0);
    load_tile(kh + (int64_t)j * KT * p.kst, vh + (int64_t)j * KT * p.kst, p.kst, tile_rows(j));
    for (int t = 0; t < n_kept; ++t) {
      __syncthreads();
      store_tile();
      __syncthreads();
      const int nrows = tile_rows(j);
      if (t + 1 < n_kept) {
        const int jn = tile_of(t + 1);
        load_tile(kh + (int64_t)jn * KT * p.kst, vh + (int64_t)jn * KT * p.kst, p.kst,
                  tile_rows(jn));
        j = jn;
      }
      if (nrows >= KT)
        compute_tile(std::false_type{}, 0ull);
      else
        compute_tile(std::true_type{}, ~0ull << nrows);
    }
  }

  // ---- phase 2: landmarks of the omitted tiles, KT per block
  if (!dense && p.top_k < p.tk) {
    const int nblk = p.tkp / KT;
    const uint16_t* kb = p.kbar_b + (int64_t)h * p.tkp * kHeadDim;
    const uint16_t* vb = p.vbar_b + (int64_t)h * p.tkp * kHeadDim;
    load_tile(kb, vb, kHeadDim, KT);
    for (int c = 0; c < nblk; ++c) {
      __syncthreads();
      store_tile();
      __syncthreads();
      if (c + 1 < nblk)
        load_tile(kb + (int64_t)(c + 1) * KT * kHeadDim, vb + (int64_t)(c + 1) * KT * kHeadDim,
                  kHeadDim, KT);
      const int j0 = c * KT;
      uint64_t kept = bitmap[j0 >> 5];
      if (KT == 64) kept |= (uint64_t)bitmap[(j0 >> 5) + 1] << 32;
      const int past = p.tk - j0;  // landmarks beyond tk are excluded
      if (past < KT) kept |= ~0ull << past;
      if (KT < 64) kept &= (1ull << KT) - 1;
      if (kept == ((KT == 64) ? ~0ull : ((1ull << KT) - 1))) continue;
      if (kept == 0ull)
        compute_tile(std::false_type{}, 0ull);
      else
        compute_tile(std::true_type{}, kept);
    }
  }

  // ---- epilogue: O / l, lane (qi, hh) holds channels 32db + 8g + 4hh + r
  const float l_tot = l_run + __shfl_xor(l_run, 32, kWave);
  const float inv = 1.0f / l_tot;
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

// fp32 landmarks -> bf16 rows [H][tkp][64], zero rows past tk.
__global__ void pack_landmarks_kernel(const float* __restrict__ kbar,
                                      const float* __restrict__ vbar, int32_t tk, int32_t tkp,
                                      int32_t heads, uint16_t* __restrict__ kb,
                                      uint16_t* __restrict__ vb) {
  const int64_t total = (int64_t)heads * tkp * (kHeadDim / 2);
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t pair = e % (kHeadDim / 2);
    const int64_t row = (e / (kHeadDim / 2)) % tkp;
    const int64_t h = e / ((int64_t)(kHeadDim / 2) * tkp);
    uint32_t wk = 0, wv = 0;
    if (row < tk) {
      const int64_t src = (h * tk + row) * kHeadDim + 2 * pair;
      wk = pack_bf16x2(kbar[src], kbar[src + 1]);
      wv = pack_bf16x2(vbar[src], vbar[src + 1]);
    }
    const int64_t dst = (h * tkp + row) * kHeadDim + 2 * pair;
    *(uint32_t*)(kb + dst) = wk;
    *(uint32_t*)(vb + dst) = wv;
  }
}

int padded_tiles(int64_t n_kv, int32_t k_tile) {
  const int64_t tk = (n_kv + k_tile - 1) / k_tile;
  return (int)(((tk + k_tile - 1) / k_tile) * k_tile);  // landmark blocks of k_tile rows
}

template <int QT, int KT>
hipError_t launch_kernel(const SparseParams& p, int heads, hipStream_t s) {
  const int64_t blocks = (int64_t)heads * p.tq;
  hipLaunchKernelGGL((tile_sparse_kernel<QT, KT>), dim3((unsigned)blocks), dim3(QT * 2), 0, s,
                     p);
  return hipGetLastError();
}

}  // namespace

size_t sparse_workspace_bytes(int64_t n_kv, int32_t heads, int32_t k_tile) {
  return (size_t)2 * heads * (size_t)padded_tiles(n_kv, k_tile) * kHeadDim * sizeof(uint16_t);
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
  p.sel = sel;
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
  p.tkp = padded_tiles(nk, k_tile);
  p.top_k = top_k;
  p.scale_log2 = scale * kLog2e;
  p.o_f32 = o_f32 ? 1 : 0;
  p.kbar_b = nullptr;
  p.vbar_b = nullptr;
  if (p.tq == 0 || heads == 0) return hipSuccess;
  if (sel != nullptr && top_k < p.tk) {
    uint16_t* kb = (uint16_t*)ws;
    uint16_t* vb = kb + (size_t)heads * p.tkp * kHeadDim;
    const int64_t total = (int64_t)heads * p.tkp * (kHeadDim / 2);
    const int blocks = (int)std::min<int64_t>((total + 255) / 256, 8192);
    hipLaunchKernelGGL(pack_landmarks_kernel, dim3(blocks), dim3(256), 0, s, kbar, vbar, p.tk,
                       p.tkp, heads, kb, vb);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    p.kbar_b = kb;
    p.vbar_b = vb;
  } else {
    p.sel = nullptr;  // every tile kept: dense attention, no landmarks
  }
  if (k_tile == 64) {
    if (q_tile == 32) return launch_kernel<32, 64>(p, heads, s);
    if (q_tile == 64) return launch_kernel<64, 64>(p, heads, s);
    return launch_kernel<128, 64>(p, heads, s);
  }
  if (q_tile == 32) return launch_kernel<32, 32>(p, heads, s);
  if (q_tile == 64) return launch_kernel<64, 32>(p, heads, s);
  return launch_kernel<128, 32>(p, heads, s);
}

}  // namespace zebra
