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
//
// bf16 with D = 128 runs decode_mfma_kernel instead: each wave takes 64 list
// entries and gathers their K and V rows into LDS with direct 16-byte loads
// (every load instruction covers 4 whole rows), then S^T = K Q^T and
// O^T += V^T P^T run on v_mfma_f32_32x32x16_bf16 with the kv head's G query
// heads as the 32 columns.  Each wave writes its own (max, sum, o) triple.
#include "lds_dma.h"

#include <algorithm>

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

// ---------------------------------------------------------------- bf16, D = 128
constexpr int kWaveKeys = 64;   // list entries per wave
constexpr int kMfmaWaves = 1;   // waves per workgroup (32 KB of LDS: five workgroups per CU)
constexpr int kDRowB = 256;     // bytes per K/V row

// chunk c of row r at c ^ (((r & 3) << 2) | ((r >> 2) & 3)): conflict-free for
// both the 16-byte row reads (S^T) and the transposing reads (O^T)
__device__ __forceinline__ int dswz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

__global__ __launch_bounds__(kMfmaWaves * 64) void decode_mfma_kernel(DmaAttnArgs a,
                                                                          int nsplit) {
  __shared__ __align__(16) unsigned char sk[kMfmaWaves][kWaveKeys * kDRowB];
  __shared__ __align__(16) unsigned char sv[kMfmaWaves][kWaveKeys * kDRowB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int G = (int)(a.Hq / a.Hkv);
  const int h = blockIdx.y, b = blockIdx.z;
  const int split = blockIdx.x * kMfmaWaves + wave;
  const int64_t seg = (int64_t)b * a.Hkv + h;
  const int cnt = a.u_cnt[seg];
  const float dmax = a.u_dmax[seg];
  const int32_t* list = a.u_idx + seg * a.u_stride;
  const int k0 = split * kWaveKeys;
  const int nk = max(0, min(kWaveKeys, cnt - k0));
  const int n = l32;  // query head column: hq = h*G + n for n < G
  float* part = static_cast<float*>(a.ws) + (((int64_t)b * a.Hq + h * G + min(n, G - 1)) * nsplit + split) * 130;
  if (nk == 0) {
    if (n < G) {
      if (hi == 0) {
        part[0] = -INFINITY;
        part[1] = 0.f;
      }
#pragma unroll
      for (int d = 0; d < 64; ++d) part[2 + hi * 64 + d] = 0.f;
    }
    return;
  }
  // list entry of this lane's key (clamped: positions past the list repeat its
  // last key and are masked)
  const int jk = list[k0 + min(lane, nk - 1)];
  const float bias = a.delta[seg * a.Sk + jk] - dmax;
  const unsigned char* Kg = static_cast<const unsigned char*>(a.K) + (b * a.ksb + h * a.ksh) * 2;
  const unsigned char* Vg = static_cast<const unsigned char*>(a.V) + (b * a.ksb + h * a.ksh) * 2;
  const uint32_t rowb = (uint32_t)(a.kss * 2);
  const uint32_t lk = dma::lds_addr(&sk[wave][0]), lv = dma::lds_addr(&sv[wave][0]);
  // 16 pieces of 4 rows: lane L fills row 4p + L/16, chunk slot L%16
#pragma unroll
  for (int p = 0; p < 16; ++p) {
    const int row = p * 4 + (lane >> 4);
    const int lc = (lane & 15) ^ dswz(row);
    const uint32_t j = (uint32_t)__shfl(jk, row);
    dma::dma_b128(Kg + j * rowb + lc * 16, lk + p * 1024);
    dma::dma_b128(Vg + j * rowb + lc * 16, lv + p * 1024);
  }
  // Q^T operands: column n (query head h*G + n; zero past G), d = kk*16 + 8*hi + [0, 8)
  dma::bf16x8 qf[8];
  {
    const uint16_t* qrow = static_cast<const uint16_t*>(a.Q) + b * a.qsb +
                           (int64_t)(h * G + min(n, G - 1)) * a.qsh;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      dma::u32x4 v = *reinterpret_cast<const dma::u32x4*>(qrow + kk * 16 + hi * 8);
      if (n >= G) v = dma::u32x4{0u, 0u, 0u, 0u};
      qf[kk] = __builtin_bit_cast(dma::bf16x8, v);
    }
  }
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0);  // this wave's rows have landed in its own LDS
  asm volatile("" ::: "memory");
  const unsigned char* KT = sk[wave];
  const unsigned char* VT = sv[wave];
  // S^T = K Q^T: register i of block mb is key mb*32 + 8(i/4) + 4hi + i%4
  dma::f32x16 s[2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) s[mb][i] = 0.f;
#pragma unroll
  for (int kk = 0; kk < 8; ++kk)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int row = mb * 32 + l32;
      const dma::bf16x8 kop = *reinterpret_cast<const dma::bf16x8*>(
          KT + row * kDRowB + (((2 * kk + hi) ^ dswz(row)) << 4));
      s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qf[kk], s[mb], 0, 0, 0);
    }
  // logits with the keys' bias; the lane's column is one query head
  float mx = -INFINITY;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = mb * 32 + 8 * (i >> 2) + 4 * hi + (i & 3);
      const float bk = __shfl(bias, key);
      const float v = key < nk ? fmaf(s[mb][i], a.scale, bk) : -INFINITY;
      s[mb][i] = v;
      mx = fmaxf(mx, v);
    }
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  // l sums the weights (the log-sum-exp); lr sums them as rounded to bf16 for
  // the PV product, which normalises this split's output, so a row dominated
  // by one key returns that key's value row unaffected by the weight's rounding
  float l = 0.f, lr = 0.f;
  dma::bf16x8 pb[2][2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      float p[8];
#pragma unroll
      for (int t8 = 0; t8 < 8; ++t8) {
        p[t8] = __expf(s[mb][hf * 8 + t8] - mx);
        l += p[t8];
      }
      pb[mb][hf] = dma::to_bf16x8(p);
#pragma unroll
      for (int t8 = 0; t8 < 8; ++t8) lr += (float)pb[mb][hf][t8];
    }
  l += __shfl_xor(l, 32);
  lr += __shfl_xor(lr, 32);
  // O^T += V^T P^T over four 16-key steps; V read with the transposing load
  dma::f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
  const int g = lane >> 4, r = lane & 15;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int k0r = mb * 32 + 16 * hf + 4 * (g >> 1) + (r >> 2);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int d0 = db * 32 + 16 * (g & 1) + 4 * (r & 3);
        const int lc = d0 >> 3, byte = (d0 & 7) * 2;
        typedef __attribute__((address_space(3))) unsigned char lds_u8;
        const lds_u8* base = (const lds_u8*)VT;
        const dma::i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (dma::lds_i16x4*)(base + k0r * kDRowB + ((lc ^ dswz(k0r)) << 4) + byte));
        const dma::i16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (dma::lds_i16x4*)(base + (k0r + 8) * kDRowB + ((lc ^ dswz(k0r + 8)) << 4) + byte));
        const dma::u32x2 lo2 = __builtin_bit_cast(dma::u32x2, lo);
        const dma::u32x2 up2 = __builtin_bit_cast(dma::u32x2, up);
        const dma::u32x4 vv = {lo2[0], lo2[1], up2[0], up2[1]};
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(dma::bf16x8, vv),
                                                        pb[mb][hf], o[db], 0, 0, 0);
      }
    }
  // this wave's (max, sum, o) for query head n: register i of block db is
  // d = db*32 + 8(i/4) + 4hi + i%4.  o is stored as l/lr times the product, so
  // that o / l, what the merge divides by, is the product over lr
  if (n < G) {
    const float f = lr > 0.f ? l / lr : 0.f;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[db][i] *= f;
    if (hi == 0) {
      part[0] = mx;
      part[1] = l;
    }
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
        for (int k = 0; k < 4; ++k) part[2 + db * 32 + 8 * q4 + 4 * hi + k] = o[db][4 * q4 + k];
  }
}

// Merge of the splits' (max, sum, o) triples of one query head: the largest
// max by a wave reduction, then each thread (one d) sums its splits eight
// loads at a time.
template <typename T, int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(DmaAttnArgs a, int nsplit) {
  __shared__ float s_M[D / 64];
  const int hq = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int G = (int)(a.Hq / a.Hkv);
  const int64_t seg = (int64_t)b * a.Hkv + hq / G;
  const float* ws = static_cast<const float*>(a.ws) + ((int64_t)b * a.Hq + hq) * nsplit * (D + 2);
  float M = -INFINITY;
  for (int s = d; s < nsplit; s += D) M = fmaxf(M, ws[s * (D + 2)]);
  M = dma::wave_max(M);
  if ((d & 63) == 0) s_M[d >> 6] = M;
  __syncthreads();
#pragma unroll
  for (int k = 0; k < D / 64; ++k) M = fmaxf(M, s_M[k]);
  float L = 0.f, o = 0.f;
  if (M != -INFINITY) {
    for (int s0 = 0; s0 < nsplit; s0 += 8) {
      float pm[8], pl[8], po[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float* part = ws + min(s0 + u, nsplit - 1) * (D + 2);
        pm[u] = part[0];
        pl[u] = part[1];
        po[u] = part[2 + d];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float f = s0 + u < nsplit ? expf(pm[u] - M) : 0.f;  // 0 for empty splits
        L = fmaf(pl[u], f, L);
        o = fmaf(po[u], f, o);
      }
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

hipError_t launch_mfma(const DmaAttnArgs& a, hipStream_t st) {
  const int nw = (int)((a.u_stride + kWaveKeys - 1) / kWaveKeys);  // splits: one per wave
  const int nwg = (nw + kMfmaWaves - 1) / kMfmaWaves;
  const int nsplit = nwg * kMfmaWaves;
  hipLaunchKernelGGL(decode_mfma_kernel, dim3((unsigned)nwg, (unsigned)a.Hkv, (unsigned)a.B),
                     dim3(kMfmaWaves * 64), 0, st, a, nsplit);
  hipLaunchKernelGGL((decode_combine_kernel<__bf16, 128>), dim3((unsigned)a.Hq, (unsigned)a.B),
                     dim3(128), 0, st, a, nsplit);
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
  // enough for either path: one split per 64-entry wave (bf16, D = 128) or per 256 entries
  const int64_t nw = (u_stride + kWaveKeys - 1) / kWaveKeys;
  const int64_t nsplit = std::max<int64_t>((nw + kMfmaWaves - 1) / kMfmaWaves * kMfmaWaves,
                                           (u_stride + kSplit - 1) / kSplit);
  return (size_t)(B * Hq * nsplit * (D + 2)) * sizeof(float);
}

hipError_t dma_launch_attn_decode(const DmaAttnArgs& a, int is_bf16, hipStream_t st) {
  // the MFMA kernel gathers key rows by 32-bit byte offsets from the (b, h)
  // base; caches whose rows lie further apart take the split kernel, whose
  // offsets are 64-bit
  const bool near = a.Sk <= 0 || (a.Sk - 1) * a.kss * 2 + 256 <= ((int64_t)1 << 32);
  if (is_bf16 && a.D == 128 && a.Hq / a.Hkv <= 32 && near) return launch_mfma(a, st);
  if (is_bf16) return a.D == 64 ? launch_g<__bf16, 64>(a, st) : launch_g<__bf16, 128>(a, st);
  return a.D == 64 ? launch_g<float, 64>(a, st) : launch_g<float, 128>(a, st);
}
