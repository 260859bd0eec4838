// Device helpers and launch declarations shared by the gfx950 kernels of the
// DMA forward.  Wavefronts are 64 lanes wide throughout.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define DMA_WAVE 64

namespace dma {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Order-preserving map of an fp32 value onto uint32: a < b  <=>  ord(a) < ord(b)
// and a == b  <=>  ord(a) == ord(b) (for non-NaN values).  -0 compares equal
// to +0, so it takes +0's code; equal weights then fall to the index part of
// the composite key below, as every other tie does.
__device__ __forceinline__ uint32_t ord32(float f) {
  uint32_t u = __float_as_uint(f);
  u = (u == 0x80000000u) ? 0u : u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Composite sort key of key j: larger key beats.  The index part makes all keys
// of one sequence distinct, equal weights going to the lower index.
__device__ __forceinline__ uint64_t key_of(float d, uint32_t j) {
  return ((uint64_t)ord32(d) << 32) | (uint64_t)(0xffffffffu - j);
}
__device__ __forceinline__ uint32_t index_of(uint64_t k) { return 0xffffffffu - (uint32_t)k; }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }
__device__ __forceinline__ int lane_id() { return __lane_id(); }
// number of set bits of m below this lane
__device__ __forceinline__ int rank_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
}

}  // namespace dma

// ---- host-side launchers (defined next to their kernels) -------------------
// Each returns hipGetLastError() after enqueueing.

// Raise the dynamic LDS limit of kernel `fn` on the current device to at
// least `bytes`.  The runtime call is made only when the limit has to grow:
// it costs host time that a chain of short launches shows as idle GPU time.
hipError_t dma_func_max_lds(const void* fn, size_t bytes);
// compute units of the current device (cached per device)
int dma_cu_count();
size_t dma_vproj_ws_bytes(int64_t M, int64_t N);
hipError_t dma_launch_vproj(const void* X, int64_t x_sb, int64_t x_ss, const void* Wv, void* V,
                            int64_t v_sb, int64_t v_ss, int64_t B, int64_t Sk, int64_t Cin,
                            int64_t N, int64_t Hkv, const float* Delta, const float* A,
                            float* delta, void* ws, hipStream_t st);
hipError_t dma_launch_fill_zero(float* p, int64_t n, hipStream_t st);
hipError_t dma_launch_weights_bwd(const void* V, int64_t B, int64_t Sk, int64_t Hkv, int64_t D,
                                  int64_t sb, int64_t ss, const float* Delta, const float* A,
                                  const float* ddelta, float* dV, float* dDelta, float* dA,
                                  float* dpre, hipStream_t st);
hipError_t dma_launch_weights(const void* V, int is_bf16, int64_t B, int64_t Sk, int64_t Hkv,
                              int64_t D, int64_t sb, int64_t ss, const float* Delta,
                              const float* A, float* delta, hipStream_t st);

struct DmaTopkArgs {
  const float* delta;
  int64_t B, Hkv, Sq, Sk, q0, w;
  int64_t n_tiles, u_stride, kt_stride;
  int32_t* evict;
  int32_t* u_idx;
  int32_t* u_cnt;
  int32_t* u_nfull;
  float* u_dmax;
  int32_t* kt_idx;
  int32_t* kt_cnt;
  void* ws;
  float* u_dlo = nullptr;  // prefill: largest delta before each tile's first row, or null
  float* u_dval = nullptr; // one row: delta of each listed key, or null
};
hipError_t dma_launch_topk_prefill(const DmaTopkArgs& a, hipStream_t st);
hipError_t dma_launch_topk_decode(const DmaTopkArgs& a, hipStream_t st);
hipError_t dma_launch_decode_append(const float* delta, int64_t BH, int64_t Sk, int64_t w,
                                   int32_t* u_idx, int32_t* u_cnt, int32_t* u_nfull,
                                   float* u_dmax, float* u_dval, hipStream_t st);
size_t dma_topk_ws_bytes(int64_t BH, int64_t Sq, int64_t Sk, int64_t w);
// this device's copy of the static mask scratch (DMA_TOPK_SCRATCH_BYTES)
hipError_t dma_topk_scratch(void** ptr);

struct DmaAttnArgs {
  const void* Q;
  const void* K;
  const void* V;
  int64_t B, Sq, Sk, Hq, Hkv, D;
  int64_t qsb, qss, qsh;  // Q strides (b, s, h)
  int64_t ksb, kss, ksh;  // K/V strides (b, s, h)
  int64_t q0, w;
  const float* delta;
  const int32_t* evict;
  const int32_t* u_idx;
  const int32_t* u_cnt;
  const int32_t* u_nfull;
  const float* u_dmax;
  const float* u_dlo = nullptr;  // bf16 prefill: largest delta before each tile's first row
  const float* u_dval = nullptr; // one row: delta of each listed key, or null
  int64_t n_tiles, u_stride;
  float scale;
  void* O;
  float* lse;
  void* ws;
  void* ores = nullptr;  // bf16 prefill only: O's rounding residual (fp32 O - bf16 O), or null
};
hipError_t dma_launch_attn_prefill_bf16(const DmaAttnArgs& a, hipStream_t st);

// Candidate lists of groups of 8 query tiles (512 rows): the keys some row of
// the group keeps, ascending, with their eviction rows (mask step T3).
void dma_cand_dims(int64_t Sq, int64_t Sk, int64_t w, int64_t* n_super, int64_t* cap);
hipError_t dma_launch_cand(const float* delta, const int32_t* evict, int64_t BH, int64_t Sk,
                           int64_t Sq, int64_t q0, int64_t w, int32_t* cj, int32_t* ce,
                           int32_t* ccnt, float* tile_dmax, hipStream_t st);

struct DmaBwdArgs {
  DmaAttnArgs f;      // forward arguments; f.O is the forward output, f.lse its log-sum-exp
  const void* dO;     // [B,Sq,Hq,D] contiguous, bf16
  float* dQ;          // [B,Sq,Hq,D] fp32
  float* dK;          // [B,Sk,Hkv,D] fp32
  float* dV;          // [B,Sk,Hkv,D] fp32
  float* ddelta;      // [B,Hkv,Sk] fp32
  // workspace
  float* Dv;          // [B,Hq,Sq]: dO . O per row
  int32_t* cj;        // candidate keys [B*Hkv, n_super, cap]
  int32_t* ce;        // their eviction rows
  int32_t* ccnt;      // [B*Hkv, n_super]
  float* cdmax;       // [B*Hkv, n_tiles] (written by the candidate kernel, unused)
  float* pk;          // dK partials [B*Hkv, n_super, cap, D]
  float* pv;          // dV partials
  float* pd;          // ddelta partials [B*Hkv, n_super, cap]
  int32_t* pmap;      // [B*Hkv, n_super, Sk]: a group's candidate position of key j
  int64_t n_super, cap;
};
size_t dma_attn_bwd_ws_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Sk,
                             int64_t w);
hipError_t dma_launch_attn_bwd(DmaBwdArgs& a, hipStream_t st);
hipError_t dma_launch_attn_prefill_f32(const DmaAttnArgs& a, hipStream_t st);
hipError_t dma_launch_attn_decode(const DmaAttnArgs& a, int is_bf16, hipStream_t st);
size_t dma_attn_decode_ws_bytes(int64_t B, int64_t Hq, int64_t D, int64_t u_stride);
