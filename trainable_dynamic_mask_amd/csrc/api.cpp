// C ABI of the DMA forward (declared in include/dma.h): host-side argument
// validation, size queries and dispatch to the gfx950 kernels.  Nothing is
// enqueued unless every argument checks out.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <map>
#include <mutex>
#include <utility>

#include "../../include/dma.h"
#include "common.h"

namespace {

constexpr int kAbiVersion = 6;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct Dims {
  int64_t n_tiles, u_stride, kt_stride;
};

// Shapes shared by the mask and attention calls.
dma_status check_mask_shape(int64_t B, int64_t Hkv, int64_t Sq, int64_t Sk, int64_t q0,
                            int64_t w) {
  if (B < 0 || Hkv < 1 || Sq < 0 || Sk < 0 || q0 < 0 || w < 1) return DMA_ERR_INVALID_ARG;
  if (q0 + Sq > Sk) return DMA_ERR_INVALID_ARG;
  if (Sk > DMA_MAX_SK) return DMA_ERR_UNSUPPORTED;
  if (B * Hkv > 65535) return DMA_ERR_UNSUPPORTED;  // (batch, kv head) is a grid dimension
  return DMA_OK;
}

Dims dims_of(int64_t Sq, int64_t Sk, int64_t w) {
  Dims d;
  d.n_tiles = cdiv(Sq, DMA_BLOCK_Q);
  d.u_stride = Sq == 1 ? (w < Sk ? w : Sk) : (w + DMA_BLOCK_Q - 1 < Sk ? w + DMA_BLOCK_Q - 1 : Sk);
  if (d.u_stride < 1) d.u_stride = 1;
  d.kt_stride = cdiv(Sk, DMA_BLOCK_K);
  if (d.kt_stride < 1) d.kt_stride = 1;
  return d;
}

dma_status hip_status(hipError_t e) { return e == hipSuccess ? DMA_OK : DMA_ERR_HIP; }

}  // namespace

hipError_t dma_func_max_lds(const void* fn, size_t bytes) {
  static std::mutex mu;
  static std::map<std::pair<const void*, int>, size_t> set;  // (kernel, device) -> limit
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  size_t& cur = set[{fn, dev}];
  if (bytes <= cur) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess) cur = bytes;
  return e;
}

int dma_cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

extern "C" {

const char* dma_status_string(dma_status s) {
  switch (s) {
    case DMA_OK: return "ok";
    case DMA_ERR_INVALID_ARG: return "invalid argument";
    case DMA_ERR_UNSUPPORTED: return "unsupported shape";
    case DMA_ERR_WORKSPACE: return "workspace too small";
    case DMA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

int dma_abi_version(void) { return kAbiVersion; }

void dma_tile_sizes(int32_t* Bq, int32_t* Bk) {
  if (Bq) *Bq = DMA_BLOCK_Q;
  if (Bk) *Bk = DMA_BLOCK_K;
}

dma_status dma_mask_dims_for(int64_t B, int64_t Hkv, int64_t Sq, int64_t Sk, int64_t q_offset,
                             int64_t w, dma_mask_dims* out) {
  if (!out) return DMA_ERR_INVALID_ARG;
  const dma_status st = check_mask_shape(B, Hkv, Sq, Sk, q_offset, w);
  if (st != DMA_OK) return st;
  const Dims d = dims_of(Sq, Sk, w);
  out->n_tiles = d.n_tiles;
  out->n_tiles_total = B * Hkv * d.n_tiles;
  out->u_stride = d.u_stride;
  out->kt_stride = d.kt_stride;
  out->evict_elems = Sq == 1 ? 0 : B * Hkv * Sk;
  out->u_elems = out->n_tiles_total * d.u_stride;
  out->kt_elems = out->n_tiles_total * d.kt_stride;
  return DMA_OK;
}

size_t dma_topk_workspace_bytes(int64_t B, int64_t Hkv, int64_t Sq, int64_t Sk, int64_t w) {
  if (B <= 0 || Hkv <= 0 || Sq <= 1 || Sk <= 0 || w <= 0) return 0;
  return dma_topk_ws_bytes(B * Hkv, Sq, Sk, w);
}

size_t dma_attn_workspace_bytes(int64_t B, int64_t Hq, int64_t Sq, int64_t D, int64_t w) {
  if (B <= 0 || Hq <= 0 || Sq != 1 || D <= 0 || w <= 0) return 0;
  return dma_attn_decode_ws_bytes(B, Hq, D, w);
}

dma_status dma_weights(const void* V, dma_dtype vt, int64_t B, int64_t Sk, int64_t Hkv, int64_t D,
                       int64_t v_stride_b, int64_t v_stride_s, const float* Delta, const float* A,
                       float* delta, void* stream) {
  if (vt != DMA_F32 && vt != DMA_BF16) return DMA_ERR_INVALID_ARG;
  if (B < 0 || Sk < 0 || Hkv < 1 || D < 1) return DMA_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return DMA_ERR_UNSUPPORTED;
  if (Hkv * D > 2048) return DMA_ERR_UNSUPPORTED;
  if (Sk > ((int64_t)1 << 31) - 64 || B > 65535) return DMA_ERR_UNSUPPORTED;
  if (B == 0 || Sk == 0) return DMA_OK;
  if (!V || !Delta || !A || !delta) return DMA_ERR_INVALID_ARG;
  const int64_t esz = vt == DMA_BF16 ? 2 : 4;
  if (v_stride_s < Hkv * D || v_stride_b < 0 || (B > 1 && v_stride_b < v_stride_s * Sk))
    return DMA_ERR_INVALID_ARG;
  if (!aligned16(V) || (v_stride_s * esz) % 16 != 0 || (v_stride_b * esz) % 16 != 0)
    return DMA_ERR_INVALID_ARG;
  return hip_status(dma_launch_weights(V, vt == DMA_BF16, B, Sk, Hkv, D, v_stride_b, v_stride_s,
                                       Delta, A, delta, static_cast<hipStream_t>(stream)));
}

size_t dma_vproj_workspace_bytes(int64_t B, int64_t Sk, int64_t Hkv, int64_t D) {
  if (B < 1 || Sk < 1 || Hkv < 1 || D < 1) return 0;
  return dma_vproj_ws_bytes(B * Sk, Hkv * D);
}

dma_status dma_vproj_weights(const void* X, int64_t B, int64_t Sk, int64_t Cin,
                             int64_t x_stride_b, int64_t x_stride_s, const void* Wv, int64_t Hkv,
                             int64_t D, void* V, int64_t v_stride_b, int64_t v_stride_s,
                             const float* Delta, const float* A, float* delta, void* ws,
                             size_t ws_bytes, void* stream) {
  if (B < 0 || Sk < 0 || Cin < 1 || Hkv < 1 || D < 1) return DMA_ERR_INVALID_ARG;
  const int64_t N = Hkv * D;
  if (Cin % 64 != 0 || N % 256 != 0 || N > 2048) return DMA_ERR_UNSUPPORTED;
  if (delta && Hkv > 8) return DMA_ERR_UNSUPPORTED;
  if (B * Sk >= ((int64_t)1 << 31) || B > 65535) return DMA_ERR_UNSUPPORTED;
  if (B == 0 || Sk == 0) return DMA_OK;
  if (!X || !Wv || !V) return DMA_ERR_INVALID_ARG;
  if (delta && (!Delta || !A)) return DMA_ERR_INVALID_ARG;
  if (x_stride_s < Cin || x_stride_b < 0 || (B > 1 && x_stride_b < x_stride_s * Sk))
    return DMA_ERR_INVALID_ARG;
  if (v_stride_s < N || v_stride_b < 0 || (B > 1 && v_stride_b < v_stride_s * Sk))
    return DMA_ERR_INVALID_ARG;
  if (!aligned16(X) || !aligned16(Wv) || !aligned16(V) || (x_stride_s * 2) % 16 != 0 ||
      (x_stride_b * 2) % 16 != 0 || (v_stride_s * 2) % 16 != 0 || (v_stride_b * 2) % 16 != 0)
    return DMA_ERR_INVALID_ARG;
  if (delta) {
    if (!ws || ws_bytes < dma_vproj_workspace_bytes(B, Sk, Hkv, D)) return DMA_ERR_WORKSPACE;
    if (!aligned16(ws)) return DMA_ERR_INVALID_ARG;
  }
  return hip_status(dma_launch_vproj(X, x_stride_b, x_stride_s, Wv, V, v_stride_b, v_stride_s, B,
                                     Sk, Cin, N, Hkv, Delta, A, delta, ws,
                                     static_cast<hipStream_t>(stream)));
}

dma_status dma_topk_mask(const float* delta, int64_t B, int64_t Hkv, int64_t Sq, int64_t Sk,
                         int64_t q_offset, int64_t w, const dma_mask* out, void* ws,
                         size_t ws_bytes, void* stream) {
  const dma_status st = check_mask_shape(B, Hkv, Sq, Sk, q_offset, w);
  if (st != DMA_OK) return st;
  if (!out) return DMA_ERR_INVALID_ARG;
  if (B == 0 || Sq == 0) return DMA_OK;
  if (!delta || !out->u_idx || !out->u_cnt || !out->u_nfull || !out->u_dmax)
    return DMA_ERR_INVALID_ARG;
  if ((out->kt_idx == nullptr) != (out->kt_cnt == nullptr)) return DMA_ERR_INVALID_ARG;
  if (Sq > 1 && !out->evict) return DMA_ERR_INVALID_ARG;
  const Dims d = dims_of(Sq, Sk, w);
  DmaTopkArgs a;
  a.delta = delta;
  a.B = B;
  a.Hkv = Hkv;
  a.Sq = Sq;
  a.Sk = Sk;
  a.q0 = q_offset;
  a.w = w;
  a.n_tiles = d.n_tiles;
  a.u_stride = d.u_stride;
  a.kt_stride = d.kt_stride;
  a.evict = out->evict;
  a.u_idx = out->u_idx;
  a.u_cnt = out->u_cnt;
  a.u_nfull = out->u_nfull;
  a.u_dmax = out->u_dmax;
  a.kt_idx = out->kt_idx;
  a.kt_cnt = out->kt_cnt;
  a.ws = ws;
  a.u_dlo = Sq > 1 ? out->u_dlo : nullptr;
  a.u_dval = Sq == 1 ? out->u_dval : nullptr;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (Sq == 1) return hip_status(dma_launch_topk_decode(a, s));
  const size_t need = dma_topk_workspace_bytes(B, Hkv, Sq, Sk, w);
  if (ws_bytes < need || !ws) return DMA_ERR_WORKSPACE;
  if (!aligned16(ws)) return DMA_ERR_INVALID_ARG;
  return hip_status(dma_launch_topk_prefill(a, s));
}

dma_status dma_topk_mask_noalloc(const float* delta, int64_t B, int64_t Hkv, int64_t Sq,
                                 int64_t Sk, int64_t q_offset, int64_t w, const dma_mask* out,
                                 void* stream) {
  const dma_status st = check_mask_shape(B, Hkv, Sq, Sk, q_offset, w);
  if (st != DMA_OK) return st;
  const size_t need = dma_topk_workspace_bytes(B, Hkv, Sq, Sk, w);
  if (need > DMA_TOPK_SCRATCH_BYTES) return DMA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0 && out && B > 0 && Sq > 0) {
    if (dma_topk_scratch(&ws) != hipSuccess) return DMA_ERR_HIP;
  }
  return dma_topk_mask(delta, B, Hkv, Sq, Sk, q_offset, w, out, ws, need, stream);
}

dma_status dma_decode_keep_append(const float* delta, int64_t B, int64_t Hkv, int64_t Sk,
                                  int64_t w, const dma_mask* mask, void* stream) {
  if (B < 0 || Hkv < 1 || w < 1 || Sk < 0) return DMA_ERR_INVALID_ARG;
  if (!mask) return DMA_ERR_INVALID_ARG;
  if (Sk - 1 < w) return DMA_ERR_INVALID_ARG;  // keep(Sk-2) must hold w keys
  if (w > 32768) return DMA_ERR_UNSUPPORTED;     // the list is staged in LDS
  if (B * Hkv > 65535) return DMA_ERR_UNSUPPORTED;
  if (mask->kt_idx || mask->kt_cnt) return DMA_ERR_INVALID_ARG;  // key-tile lists are not kept
  if (B == 0) return DMA_OK;
  if (!delta || !mask->u_idx || !mask->u_cnt || !mask->u_nfull || !mask->u_dmax)
    return DMA_ERR_INVALID_ARG;
  return hip_status(dma_launch_decode_append(delta, B * Hkv, Sk, w, mask->u_idx, mask->u_cnt,
                                             mask->u_nfull, mask->u_dmax, mask->u_dval,
                                             static_cast<hipStream_t>(stream)));
}

namespace {
dma_status attn_fwd_impl(const void* Q, const void* K, const void* V, dma_dtype t, int64_t B,
                         int64_t Sq, int64_t Sk, int64_t Hq, int64_t Hkv, int64_t D,
                         const int64_t q_strides[3], const int64_t kv_strides[3],
                         int64_t q_offset, int64_t w, const float* delta, const dma_mask* mask,
                         float scale, void* O, float* lse, void* O_res, void* ws,
                         size_t ws_bytes, void* stream) {
  if (t != DMA_F32 && t != DMA_BF16) return DMA_ERR_INVALID_ARG;
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || D < 1) return DMA_ERR_INVALID_ARG;
  const dma_status st = check_mask_shape(B, Hkv, Sq, Sk, q_offset, w);
  if (st != DMA_OK) return st;
  if (D != 64 && D != 128) return DMA_ERR_UNSUPPORTED;
  if (t == DMA_BF16 && Sq > 1 && D != 128) return DMA_ERR_UNSUPPORTED;
  if (std::isnan(scale)) return DMA_ERR_INVALID_ARG;
  if (B == 0 || Sq == 0) return DMA_OK;
  if (!Q || !K || !V || !delta || !mask || !O || !q_strides || !kv_strides)
    return DMA_ERR_INVALID_ARG;
  if (!mask->u_idx || !mask->u_cnt || !mask->u_nfull || !mask->u_dmax) return DMA_ERR_INVALID_ARG;
  if (Sq > 1 && !mask->evict) return DMA_ERR_INVALID_ARG;
  if (Sq > 1 && t == DMA_BF16 && !mask->u_dlo) return DMA_ERR_INVALID_ARG;
  const int64_t esz = t == DMA_BF16 ? 2 : 4;
  for (int i = 0; i < 3; ++i)
    if (q_strides[i] < 0 || kv_strides[i] < 0 || (q_strides[i] * esz) % 16 != 0 ||
        (kv_strides[i] * esz) % 16 != 0)
      return DMA_ERR_INVALID_ARG;
  if ((Hq > 1 && q_strides[2] < D) || (Hkv > 1 && kv_strides[2] < D)) return DMA_ERR_INVALID_ARG;
  // the bf16 prefill gathers key rows by 32-bit byte offsets from the (b, h)
  // base, formed by 24-bit products of key index and row stride
  if (t == DMA_BF16 && Sq > 1 && Sk > 0 &&
      ((Sk - 1) * kv_strides[1] * 2 + 256 > ((int64_t)1 << 32) ||
       kv_strides[1] * 2 >= ((int64_t)1 << 24) || Sk > ((int64_t)1 << 24)))
    return DMA_ERR_UNSUPPORTED;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O)) return DMA_ERR_INVALID_ARG;
  const Dims d = dims_of(Sq, Sk, w);
  DmaAttnArgs a;
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.B = B;
  a.Sq = Sq;
  a.Sk = Sk;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.D = D;
  a.qsb = q_strides[0];
  a.qss = q_strides[1];
  a.qsh = q_strides[2];
  a.ksb = kv_strides[0];
  a.kss = kv_strides[1];
  a.ksh = kv_strides[2];
  a.q0 = q_offset;
  a.w = w;
  a.delta = delta;
  a.evict = mask->evict;
  a.u_idx = mask->u_idx;
  a.u_cnt = mask->u_cnt;
  a.u_nfull = mask->u_nfull;
  a.u_dmax = mask->u_dmax;
  a.u_dlo = mask->u_dlo;
  a.u_dval = Sq == 1 ? mask->u_dval : nullptr;
  a.n_tiles = d.n_tiles;
  a.u_stride = d.u_stride;
  a.scale = scale > 0.f ? scale : 1.f / std::sqrt((float)D);
  a.O = O;
  a.lse = lse;
  a.ws = ws;
  a.ores = O_res;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (Sq == 1) {
    const size_t need = dma_attn_decode_ws_bytes(B, Hq, D, d.u_stride);
    if (ws_bytes < need || !ws) return DMA_ERR_WORKSPACE;
    if (!aligned16(ws)) return DMA_ERR_INVALID_ARG;
    return hip_status(dma_launch_attn_decode(a, t == DMA_BF16, s));
  }
  if (t == DMA_BF16) return hip_status(dma_launch_attn_prefill_bf16(a, s));
  return hip_status(dma_launch_attn_prefill_f32(a, s));
}
}  // namespace

dma_status dma_attn_fwd(const void* Q, const void* K, const void* V, dma_dtype t, int64_t B,
                        int64_t Sq, int64_t Sk, int64_t Hq, int64_t Hkv, int64_t D,
                        const int64_t q_strides[3], const int64_t kv_strides[3], int64_t q_offset,
                        int64_t w, const float* delta, const dma_mask* mask, float scale, void* O,
                        float* lse, void* ws, size_t ws_bytes, void* stream) {
  return attn_fwd_impl(Q, K, V, t, B, Sq, Sk, Hq, Hkv, D, q_strides, kv_strides, q_offset, w,
                       delta, mask, scale, O, lse, nullptr, ws, ws_bytes, stream);
}

dma_status dma_attn_fwd_train(const void* Q, const void* K, const void* V, dma_dtype t,
                              int64_t B, int64_t Sq, int64_t Sk, int64_t Hq, int64_t Hkv,
                              int64_t D, const int64_t q_strides[3],
                              const int64_t kv_strides[3], int64_t q_offset, int64_t w,
                              const float* delta, const dma_mask* mask, float scale, void* O,
                              float* lse, void* O_res, void* stream) {
  if (t != DMA_BF16 || D != 128 || Sq == 1) return DMA_ERR_UNSUPPORTED;
  if (B > 0 && Sq > 0 && (!lse || !O_res || !aligned16(O_res))) return DMA_ERR_INVALID_ARG;
  return attn_fwd_impl(Q, K, V, t, B, Sq, Sk, Hq, Hkv, D, q_strides, kv_strides, q_offset, w,
                       delta, mask, scale, O, lse, O_res, nullptr, 0, stream);
}

size_t dma_weights_bwd_workspace_bytes(int64_t B, int64_t Sk, int64_t Hkv) {
  if (B <= 0 || Sk <= 0 || Hkv <= 0) return 0;
  return (size_t)(B * Sk * Hkv) * sizeof(float);
}

dma_status dma_weights_bwd(const void* V, dma_dtype vt, int64_t B, int64_t Sk, int64_t Hkv,
                           int64_t D, int64_t v_stride_b, int64_t v_stride_s, const float* Delta,
                           const float* A, const float* ddelta, float* dV, float* dDelta,
                           float* dA, void* ws, size_t ws_bytes, void* stream) {
  if (vt != DMA_F32 && vt != DMA_BF16) return DMA_ERR_INVALID_ARG;
  if (B < 0 || Sk < 0 || Hkv < 1 || D < 1) return DMA_ERR_INVALID_ARG;
  if (vt != DMA_BF16 || (D != 64 && D != 128)) return DMA_ERR_UNSUPPORTED;
  if (Hkv * D > 2048) return DMA_ERR_UNSUPPORTED;
  if (Sk > ((int64_t)1 << 31) - 64 || B > 65535) return DMA_ERR_UNSUPPORTED;
  if (!Delta || !A || !dDelta || !dA) return DMA_ERR_INVALID_ARG;
  if (v_stride_s < Hkv * D || v_stride_b < 0 || (B > 1 && v_stride_b < v_stride_s * Sk))
    return DMA_ERR_INVALID_ARG;
  if (B == 0 || Sk == 0) {
    // no keys: the gradients of Delta and A are zero
    hipStream_t s = static_cast<hipStream_t>(stream);
    dma_launch_fill_zero(dDelta, Hkv * D * Hkv, s);
    return hip_status(dma_launch_fill_zero(dA, Hkv, s));
  }
  if (!V || !ddelta || !dV) return DMA_ERR_INVALID_ARG;
  if (!aligned16(V) || (v_stride_s * 2) % 16 != 0 || (v_stride_b * 2) % 16 != 0)
    return DMA_ERR_INVALID_ARG;
  if (ws_bytes < dma_weights_bwd_workspace_bytes(B, Sk, Hkv) || !ws) return DMA_ERR_WORKSPACE;
  if (!aligned16(ws)) return DMA_ERR_INVALID_ARG;
  return hip_status(dma_launch_weights_bwd(V, B, Sk, Hkv, D, v_stride_b, v_stride_s, Delta, A,
                                           ddelta, dV, dDelta, dA, static_cast<float*>(ws),
                                           static_cast<hipStream_t>(stream)));
}

size_t dma_attn_bwd_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Sk,
                                    int64_t w) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Sq <= 1 || Sk <= 0 || w <= 0) return 0;
  return dma_attn_bwd_ws_bytes(B, Hq, Hkv, Sq, Sk, w);
}

dma_status dma_attn_bwd(const void* Q, const void* K, const void* V, dma_dtype t, int64_t B,
                        int64_t Sq, int64_t Sk, int64_t Hq, int64_t Hkv, int64_t D,
                        const int64_t q_strides[3], const int64_t kv_strides[3], int64_t q_offset,
                        int64_t w, const float* delta, const dma_mask* mask, float scale,
                        const void* O, const void* O_res, const float* lse, const void* dO,
                        float* dQ, float* dK, float* dV, float* ddelta, void* ws,
                        size_t ws_bytes, void* stream) {
  if (t != DMA_F32 && t != DMA_BF16) return DMA_ERR_INVALID_ARG;
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || D < 1) return DMA_ERR_INVALID_ARG;
  const dma_status st = check_mask_shape(B, Hkv, Sq, Sk, q_offset, w);
  if (st != DMA_OK) return st;
  if (t != DMA_BF16 || D != 128 || Sq == 1) return DMA_ERR_UNSUPPORTED;
  if (std::isnan(scale)) return DMA_ERR_INVALID_ARG;
  if (B == 0 || Sq == 0) return DMA_OK;
  if (!Q || !K || !V || !delta || !mask || !O || !lse || !dO || !dQ || !dK || !dV || !ddelta ||
      !q_strides || !kv_strides)
    return DMA_ERR_INVALID_ARG;
  if (!mask->evict || !mask->u_idx || !mask->u_cnt || !mask->u_nfull || !mask->u_dmax)
    return DMA_ERR_INVALID_ARG;
  for (int i = 0; i < 3; ++i)
    if (q_strides[i] < 0 || kv_strides[i] < 0 || (q_strides[i] * 2) % 16 != 0 ||
        (kv_strides[i] * 2) % 16 != 0)
      return DMA_ERR_INVALID_ARG;
  if ((Hq > 1 && q_strides[2] < D) || (Hkv > 1 && kv_strides[2] < D)) return DMA_ERR_INVALID_ARG;
  // key rows, query rows and dO rows are addressed by 32-bit byte offsets
  const int64_t lim = (int64_t)1 << 32;
  if ((Sk - 1) * kv_strides[1] * 2 + 256 > lim || (Sq - 1) * q_strides[1] * 2 + 256 > lim ||
      (Sq - 1) * Hq * D * 2 + 256 > lim)
    return DMA_ERR_UNSUPPORTED;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(dO) ||
      !aligned16(dQ) || !aligned16(dK) || !aligned16(dV) || (O_res && !aligned16(O_res)))
    return DMA_ERR_INVALID_ARG;
  const size_t need = dma_attn_bwd_ws_bytes(B, Hq, Hkv, Sq, Sk, w);
  if (ws_bytes < need || !ws) return DMA_ERR_WORKSPACE;
  if (((uintptr_t)ws & 255) != 0) return DMA_ERR_INVALID_ARG;
  const Dims d = dims_of(Sq, Sk, w);
  DmaBwdArgs a{};
  DmaAttnArgs& f = a.f;
  f.Q = Q;
  f.K = K;
  f.V = V;
  f.B = B;
  f.Sq = Sq;
  f.Sk = Sk;
  f.Hq = Hq;
  f.Hkv = Hkv;
  f.D = D;
  f.qsb = q_strides[0];
  f.qss = q_strides[1];
  f.qsh = q_strides[2];
  f.ksb = kv_strides[0];
  f.kss = kv_strides[1];
  f.ksh = kv_strides[2];
  f.q0 = q_offset;
  f.w = w;
  f.delta = delta;
  f.evict = mask->evict;
  f.u_idx = mask->u_idx;
  f.u_cnt = mask->u_cnt;
  f.u_nfull = mask->u_nfull;
  f.u_dmax = mask->u_dmax;
  f.n_tiles = d.n_tiles;
  f.u_stride = d.u_stride;
  f.scale = scale > 0.f ? scale : 1.f / std::sqrt((float)D);
  f.O = const_cast<void*>(O);
  f.lse = const_cast<float*>(lse);
  f.ws = ws;
  f.ores = const_cast<void*>(O_res);
  a.dO = dO;
  a.dQ = dQ;
  a.dK = dK;
  a.dV = dV;
  a.ddelta = ddelta;
  return hip_status(dma_launch_attn_bwd(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
