// Masked attention of the DMA forward for one query row per sequence (decode
// against a cache; Hugging Face blog "Trainable Dynamic Mask Sparse
// Attention", sections "Efficient Sparse Attention Computation" and
// "Unified Training-Inference Architecture").  The row keeps w keys out of
// the whole cache; only those K/V rows are read, so the step is bound by the
// HBM gather of 2*w*D values per (batch, kv head).
//
// Split-K: workgroup (split s, kv head, batch x head group) takes list
// entries [s*256, s*256+256) for the GB query heads of one kv head:
//   phase 1  one key per thread: K row gathered (16-byte loads), GB dot products;
//   phase 2  one wave per head: max and exp over the split's 256 scores;
//   phase 3  threads own a pair of d and a quarter of the keys: V rows are read
//            coalesced, partial sums are reduced through LDS.
// A second kernel merges the splits' (max, sum, o) triples per query head.
#include "common.h"

namespace {

constexpr int kSplit = 256;
constexpr int kThreads = 256;
constexpr int kMaxGB = 8;

template <typename T>
struct Row;
template <>
struct Row<float> {
  __device__ static float get(const float* p, int d) { return p[d]; }
};
template <>
struct Row<__bf16> {
  __device__ static float get(const __bf16* p, int d) { return (float)p[d]; }
};

template <typename T, int D, int GB>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(DmaAttnArgs a, int nsplit) {
  __shared__ float qs[GB][D];
  __shared__ float sc[GB][kSplit];
  __shared__ int js[kSplit];
  __shared__ float red[kThreads / (D / 2)][GB][D];
  __shared__ float s_m[GB], s_l[GB];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = (int)(a.Hq / a.Hkv);
  const int ngrp = G / GB;
  const int s = blockIdx.x, h = blockIdx.y;
  const int b = blockIdx.z / ngrp, hgrp = blockIdx.z % ngrp;
  const int hq0 = h * G + hgrp * GB;
  const int64_t seg = (int64_t)b * a.Hkv + h;
  const int cnt = a.u_cnt[seg];
  const float dmax = a.u_dmax[seg];
  const int32_t* list = a.u_idx + seg * a.u_stride;
  const float* dl = a.delta + seg * a.Sk;
  const T* Kg = static_cast<const T*>(a.K) + b * a.ksb + h * a.ksh;
  const T* Vg = static_cast<const T*>(a.V) + b * a.ksb + h * a.ksh;
  const int k0 = s * kSplit;
  const int nk = max(0, min(kSplit, cnt - k0));

  for (int u = tid; u < GB * D; u += kThreads) {
    const int gq = u / D, d = u % D;
    const T* qrow = static_cast<const T*>(a.Q) + b * a.qsb + (hq0 + gq) * a.qsh;
    qs[gq][d] = Row<T>::get(qrow, d);
  }
  __syncthreads();

  // phase 1: scores, one key per thread
  if (tid < nk) {
    const int j = list[k0 + tid];
    js[tid] = j;
    const T* krow = Kg + (int64_t)j * a.kss;
    float dot[GB];
#pragma unroll
    for (int gq = 0; gq < GB; ++gq) dot[gq] = 0.f;
    constexpr int E = 16 / sizeof(T);
#pragma unroll 4
    for (int d0 = 0; d0 < D; d0 += E) {
      const uint4 raw = *reinterpret_cast<const uint4*>(krow + d0);
      float kv[E];
      if constexpr (sizeof(T) == 2) {
        const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kv[2 * e] = dma::bf16_lo(w4[e]);
          kv[2 * e + 1] = dma::bf16_hi(w4[e]);
        }
      } else {
        kv[0] = __uint_as_float(raw.x);
        kv[1] = __uint_as_float(raw.y);
        kv[2] = __uint_as_float(raw.z);
        kv[3] = __uint_as_float(raw.w);
      }
#pragma unroll
      for (int gq = 0; gq < GB; ++gq)
#pragma unroll
        for (int e = 0; e < E; ++e) dot[gq] = fmaf(qs[gq][d0 + e], kv[e], dot[gq]);
    }
    const float bias = dl[j] - dmax;
#pragma unroll
    for (int gq = 0; gq < GB; ++gq) sc[gq][tid] = fmaf(dot[gq], a.scale, bias);
  }
  __syncthreads();

  // phase 2: per-head max and exponentials
  for (int gq = wave; gq < GB; gq += kThreads / 64) {
    float mx = -INFINITY;
    for (int k = lane; k < nk; k += 64) mx = fmaxf(mx, sc[gq][k]);
    mx = dma::wave_max(mx);
    float sum = 0.f;
    for (int k = lane; k < nk; k += 64) {
      const float p = expf(sc[gq][k] - mx);
      sc[gq][k] = p;
      sum += p;
    }
    sum = dma::wave_sum(sum);
    if (lane == 0) {
      s_m[gq] = mx;
      s_l[gq] = sum;
    }
  }
  __syncthreads();

  // phase 3: weighted V sum; thread owns d pair dp and key group kg
  constexpr int NDP = D / 2;
  constexpr int NKG = kThreads / NDP;
  const int dp = tid % NDP, kg = tid / NDP;
  float acc[GB][2];
#pragma unroll
  for (int gq = 0; gq < GB; ++gq) acc[gq][0] = acc[gq][1] = 0.f;
  for (int k = kg; k < nk; k += NKG) {
    const T* vrow = Vg + (int64_t)js[k] * a.kss + 2 * dp;
    const float v0 = Row<T>::get(vrow, 0), v1 = Row<T>::get(vrow, 1);
#pragma unroll
    for (int gq = 0; gq < GB; ++gq) {
      const float p = sc[gq][k];
      acc[gq][0] = fmaf(p, v0, acc[gq][0]);
      acc[gq][1] = fmaf(p, v1, acc[gq][1]);
    }
  }
#pragma unroll
  for (int gq = 0; gq < GB; ++gq) {
    red[kg][gq][2 * dp] = acc[gq][0];
    red[kg][gq][2 * dp + 1] = acc[gq][1];
  }
  __syncthreads();
  float* ws = static_cast<float*>(a.ws);
  for (int u = tid; u < GB * D; u += kThreads) {
    const int gq = u / D, d = u % D;
    float o = 0.f;
#pragma unroll
    for (int k = 0; k < NKG; ++k) o += red[k][gq][d];
    float* part = ws + (((int64_t)b * a.Hq + hq0 + gq) * nsplit + s) * (D + 2);
    part[2 + d] = o;
    if (d == 0) {
      part[0] = nk > 0 ? s_m[gq] : -INFINITY;
      part[1] = nk > 0 ? s_l[gq] : 0.f;
    }
  }
}

template <typename T, int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(DmaAttnArgs a, int nsplit) {
  const int hq = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int G = (int)(a.Hq / a.Hkv);
  const int64_t seg = (int64_t)b * a.Hkv + hq / G;
  const float* ws = static_cast<const float*>(a.ws) + ((int64_t)b * a.Hq + hq) * nsplit * (D + 2);
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, ws[s * (D + 2)]);
  float L = 0.f, o = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < nsplit; ++s) {
      const float* part = ws + s * (D + 2);
      const float f = expf(part[0] - M);  // 0 for empty splits
      L = fmaf(part[1], f, L);
      o = fmaf(part[2 + d], f, o);
    }
  }
  const float out = L > 0.f ? o / L : 0.f;
  T* orow = static_cast<T*>(a.O) + ((int64_t)b * a.Sq * a.Hq + hq) * D;
  orow[d] = (T)out;
  if (a.lse && d == 0) a.lse[(int64_t)b * a.Hq + hq] = M + logf(L) + a.u_dmax[seg];
}

template <typename T, int D, int GB>
hipError_t launch(const DmaAttnArgs& a, hipStream_t st) {
  const int G = (int)(a.Hq / a.Hkv);
  const int nsplit = (int)((a.u_stride + kSplit - 1) / kSplit);
  hipLaunchKernelGGL((decode_split_kernel<T, D, GB>),
                     dim3(nsplit, (unsigned)a.Hkv, (unsigned)(a.B * (G / GB))), dim3(kThreads), 0,
                     st, a, nsplit);
  hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3((unsigned)a.Hq, (unsigned)a.B), dim3(D),
                     0, st, a, nsplit);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_g(const DmaAttnArgs& a, hipStream_t st) {
  const int G = (int)(a.Hq / a.Hkv);
  if (G % 8 == 0) return launch<T, D, 8>(a, st);
  if (G % 4 == 0) return launch<T, D, 4>(a, st);
  if (G % 2 == 0) return launch<T, D, 2>(a, st);
  return launch<T, D, 1>(a, st);
}

}  // namespace

size_t dma_attn_decode_ws_bytes(int64_t B, int64_t Hq, int64_t D, int64_t u_stride) {
  const int64_t nsplit = (u_stride + kSplit - 1) / kSplit;
  return (size_t)(B * Hq * nsplit * (D + 2)) * sizeof(float);
}

hipError_t dma_launch_attn_decode(const DmaAttnArgs& a, int is_bf16, hipStream_t st) {
  if (is_bf16) return a.D == 64 ? launch_g<__bf16, 64>(a, st) : launch_g<__bf16, 128>(a, st);
  return a.D == 64 ? launch_g<float, 64>(a, st) : launch_g<float, 128>(a, st);
}
