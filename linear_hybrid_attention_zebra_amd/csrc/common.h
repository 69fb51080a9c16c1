// Internal helpers shared by the gfx950 kernels of libzebra (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace zebra {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kHeadDim = 64;

// bf16 stored in the high or low half of a 32-bit word -> float (exact).
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> two bf16 in one word (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 v = {a, b};
  bf16x2 r = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 w) { return __builtin_bit_cast(bf16x8, w); }

// 32x32x16 bf16 MFMA: D = A(32x16) B(16x32) + C. Lane l holds A[l%32][8(l/32)..+7],
// B[8(l/32)..+7][l%32]; D[i][l%32] with i = 8(v/4) + 4(l/32) + v%4 in register v.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ int wave_sum_int(int v) {
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Order-preserving map float -> uint32 (larger float -> larger key); -0 maps like +0.
__device__ __forceinline__ uint32_t float_key(float f) {
  if (f == 0.0f) f = 0.0f;
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace zebra

// Host-side launch helpers (defined in the kernel sources, called by zebra_abi.cpp).
namespace zebra {
struct SeqDesc {
  const void* ptr;
  int64_t n;
  int32_t heads;
  int64_t st;  // token stride (elements)
  int64_t sh;  // head stride (elements)
};

hipError_t launch_pool(const uint16_t* x, int64_t n, int32_t heads, int64_t st, int64_t sh,
                       int32_t tile, float* out, hipStream_t s);
// Row stride (floats) of the select workspace's score matrix: t_k rounded up
// to a multiple of 32, so every row starts on a 128-byte line.
inline int32_t score_row_stride(int32_t tk) { return (tk + 31) & ~31; }
hipError_t launch_select(const float* qbar, const float* kbar, int32_t heads, int32_t tq,
                         int32_t tk, int32_t top_k, int32_t* sel, float* scores,
                         hipStream_t s);
size_t sparse_workspace_bytes(int64_t n_q, int64_t n_kv, int32_t heads, int32_t q_tile,
                              int32_t k_tile, int32_t top_k);
// launch_tile_sparse flags (the same bits as the ABI's ZEBRA_SPARSE_*)
constexpr uint32_t kSparseNoLandmarks = 1u;
constexpr uint32_t kSparseLandmarkLogCount = 2u;
hipError_t launch_tile_sparse(const uint16_t* q, int64_t nq, int64_t qst, int64_t qsh,
                              const uint16_t* k, const uint16_t* v, int64_t nk, int64_t kst,
                              int64_t ksh, int32_t heads, const float* kbar, const float* vbar,
                              const int32_t* sel, int32_t q_tile, int32_t k_tile,
                              int32_t top_k, float scale, void* o, int64_t ost, int64_t osh,
                              bool o_f32, uint32_t flags, void* ws, hipStream_t s,
                              float* lse = nullptr);
// float32 landmarks [H][tk][64] -> bf16 rows (the attention kernels' operand copies)
hipError_t launch_pack_landmarks(const float* kbar, const float* vbar, int32_t heads, int32_t tk,
                                 uint16_t* kb, uint16_t* vb, hipStream_t s);
size_t sparse_bwd_workspace_bytes(int64_t n_q, int64_t n_kv, int32_t heads, int32_t q_tile,
                                  int32_t k_tile, int32_t top_k);
hipError_t launch_tile_sparse_bwd(const uint16_t* q, int64_t nq, int64_t qst, int64_t qsh,
                                  const uint16_t* k, const uint16_t* v, int64_t nk, int64_t kst,
                                  int64_t ksh, int32_t heads, const float* kbar,
                                  const float* vbar, const int32_t* sel, int32_t q_tile,
                                  int32_t k_tile, int32_t top_k, float scale, uint32_t flags,
                                  const void* dout, int64_t dst, int64_t dsh, bool g_f32,
                                  void* dq, int64_t qgst, int64_t qgsh, void* dk, void* dv,
                                  int64_t kgst, int64_t kgsh, void* ws, hipStream_t s,
                                  const float* lse_in = nullptr, const float* out_in = nullptr,
                                  int64_t ost_in = 0, int64_t osh_in = 0);
size_t linear_workspace_bytes(int64_t n_kv, int32_t heads);
// forward state S, z of every head into the linear workspace ([H][S | z] float32)
hipError_t launch_linear_state(const uint16_t* k, const uint16_t* v, int64_t nk, int64_t kst,
                               int64_t ksh, int32_t heads, void* ws, float** state_out,
                               hipStream_t s);
size_t linear_bwd_workspace_bytes(int64_t n_q, int64_t n_kv, int32_t heads);
hipError_t launch_linear_bwd(const uint16_t* q, int64_t nq, int64_t qst, int64_t qsh,
                             const uint16_t* k, const uint16_t* v, int64_t nk, int64_t kst,
                             int64_t ksh, int32_t heads, const float* aff_scale,
                             const void* dout, int64_t dst, int64_t dsh, void* dq, int64_t qgst,
                             int64_t qgsh, void* dk, void* dv, int64_t kgst, int64_t kgsh,
                             bool g_f32, float* d_scale, float* d_bias, void* ws,
                             hipStream_t s);
hipError_t launch_linear(const uint16_t* q, int64_t nq, int64_t qst, int64_t qsh,
                         const uint16_t* k, const uint16_t* v, int64_t nk, int64_t kst,
                         int64_t ksh, int32_t heads, const float* aff_scale,
                         const float* aff_bias, void* o, int64_t ost, int64_t osh, bool o_f32,
                         void* ws, hipStream_t s);
size_t mass_workspace_bytes(int64_t n_q, int32_t heads);
hipError_t launch_block_mass(const uint16_t* q, int64_t nq, int64_t qst, int64_t qsh,
                             const uint16_t* k, int64_t nk, int64_t kst, int64_t ksh,
                             int32_t heads, int32_t q_tile, int32_t k_tile, float scale,
                             float* mass, void* ws, hipStream_t s);
int64_t spatial_order(int32_t n_views, int32_t n_special, int32_t grid_h, int32_t grid_w,
                      int32_t block, int32_t* out);
hipError_t launch_permute(const void* src, int64_t s_tok, int64_t s_head, void* dst,
                          int64_t d_tok, int64_t d_head, const int32_t* order, int64_t n,
                          int32_t heads, int32_t elem_bytes, bool scatter, hipStream_t s);
hipError_t launch_fit(const float* x, const float* y, int32_t m, int32_t heads, float* a,
                      float* b, int32_t* n_deg, bool centred, hipStream_t s);
// Size of the fixed device scratch of the allocation-free linear-attention
// entry point (40 MiB: the linear workspace of up to 840 heads at any length).
constexpr size_t kNoAllocScratchBytes = size_t(40) << 20;
// The current device's scratch array (device address, taken once per device).
hipError_t noalloc_scratch(void** out);
}  // namespace zebra
