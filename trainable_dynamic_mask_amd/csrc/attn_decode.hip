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
// bf16 with D = 128 runs decode_mfma_kernel instead: each wave takes up to
// 512 list entries in 32-key stages, two stages of K and V rows in flight
// into LDS (direct 16-byte loads, every instruction 4 whole rows) while the
// previous one is computed; S^T = K Q^T and O^T += V^T P^T run on
// v_mfma_f32_32x32x16_bf16 with the kv head's G query heads as the 32
// columns.  Each wave writes one (max, sum, o) triple per query head.
#include "lds_dma.h"

#include <algorithm>
#include <type_traits>

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
    const float bias = (a.u_dval ? a.u_dval[seg * a.u_stride + k0 + tid] : dl[j]) - dmax;
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
constexpr int kStageKeys = 32;                 // list entries per pipeline stage
constexpr int kDRowB = 256;                    // bytes per K/V row
constexpr int kStageBytes = kStageKeys * kDRowB;
constexpr int kMaxStages = 16;                 // list entries per wave: at most 512
constexpr int kMinRange = 64;                  // and at least 64 (the workspace's split count)
constexpr int kPipeWavesPerCU = 5;             // 32 KB of LDS per wave

// chunk c of row r at c ^ (((r & 3) << 2) | ((r >> 2) & 3)): conflict-free for
// both the 16-byte row reads (S^T) and the transposing reads (O^T)
__device__ __forceinline__ int dswz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

// One wave per workgroup takes `range` consecutive list entries of one
// (batch, kv head) in stages of 32 keys, two stages in flight: the K and V
// rows of stage s+2 are gathered into LDS (direct 16-byte loads, 4 whole rows
// per instruction) while stage s+1's are still arriving and stage s is
// computed, so every wave keeps loads in flight from its first stage to its
// last.  S^T = K Q^T and O^T += V^T P^T run on v_mfma_f32_32x32x16_bf16 with
// the kv head's G query heads as the 32 columns; the softmax is online over
// the stages (running max per column, sums and output rescaled when it grows).
// Each wave ends with one (max, sum, o) triple per query head.  FUSED: the
// workgroup holds all nsplit waves of one (batch, kv head), which merge their
// triples through LDS and write O; otherwise one wave per workgroup writes
// its triples to the workspace for decode_combine_kernel.
template <bool FUSED>
__global__ __launch_bounds__(FUSED ? kPipeWavesPerCU * 64 : 64, 2) void decode_mfma_kernel(
    DmaAttnArgs a, int nsplit, int range) {
  extern __shared__ __align__(16) unsigned char s_dyn[];  // per wave: K[2], V[2] stages
  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31, hi = lane >> 5;
  const int G = (int)(a.Hq / a.Hkv);
  const int wave = FUSED ? __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6) : 0;
  unsigned char* const s_wave = s_dyn + wave * 4 * kStageBytes;
  unsigned char (*const sk)[kStageBytes] = reinterpret_cast<unsigned char (*)[kStageBytes]>(s_wave);
  unsigned char (*const sv)[kStageBytes] =
      reinterpret_cast<unsigned char (*)[kStageBytes]>(s_wave + 2 * kStageBytes);
  const int split = FUSED ? wave : (int)blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int64_t seg = (int64_t)b * a.Hkv + h;
  const int cnt = a.u_cnt[seg];
  const float dmax = a.u_dmax[seg];
  const int32_t* list = a.u_idx + seg * a.u_stride;
  const int k0 = split * range;
  const int nk = max(0, min(range, cnt - k0));
  const int n = l32;  // query head column: hq = h*G + n for n < G
  // running max of the lane's column, sums of the weights (l) and of the
  // weights as rounded to bf16 for the PV product (lr), both over this lane's
  // half of each stage's keys; o = O^T for the column (all empty: no keys)
  float m = -INFINITY, l = 0.f, lr = 0.f;
  dma::f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
  if (nk > 0) {
    const int nst = (nk + kStageKeys - 1) / kStageKeys;
    // list entries (and their logit biases) of the range, entry k0 + 64i + lane
    // in register i; positions past the range repeat its last entry and are
    // masked (loaded unconditionally: no branch between the loads and their use)
    int jk[kMaxStages / 2];
#pragma unroll
    for (int i = 0; i < kMaxStages / 2; ++i) jk[i] = list[k0 + min(64 * i + lane, nk - 1)];
    float bias[kMaxStages / 2];
    if (a.u_dval) {  // the mask's copy of delta at the listed keys: one contiguous read
      const float* dv = a.u_dval + seg * a.u_stride + k0;
#pragma unroll
      for (int i = 0; i < kMaxStages / 2; ++i) bias[i] = dv[min(64 * i + lane, nk - 1)] - dmax;
    } else {
#pragma unroll
      for (int i = 0; i < kMaxStages / 2; ++i) bias[i] = a.delta[seg * a.Sk + jk[i]] - dmax;
    }
    const unsigned char* Kg = static_cast<const unsigned char*>(a.K) + (b * a.ksb + h * a.ksh) * 2;
    const unsigned char* Vg = static_cast<const unsigned char*>(a.V) + (b * a.ksb + h * a.ksh) * 2;
    const uint32_t rowb = (uint32_t)(a.kss * 2);
    const uint32_t lk = dma::lds_addr(&sk[0][0]), lv = dma::lds_addr(&sv[0][0]);
    // a stage of parity P (its rows in lanes 32P.. of a jk register) into
    // buffer P: 8 pieces of 4 rows for K and for V; lane L fills row 4p + L/16,
    // chunk slot L%16
    auto issue = [&](const int jr, auto P) {
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        const int row = p * 4 + (lane >> 4);
        const int lc = (lane & 15) ^ dswz(row);
        const uint32_t j = (uint32_t)__shfl(jr, 32 * P() + row);
        dma::dma_b128_u(Kg + j * rowb + lc * 16, lk + P() * kStageBytes + p * 1024);
        dma::dma_b128_u(Vg + j * rowb + lc * 16, lv + P() * kStageBytes + p * 1024);
      }
    };
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    issue(jk[0], P0{});
    if (nst > 1) issue(jk[0], P1{});
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
    const int g = lane >> 4, r = lane & 15;
    // stage s (parity P): its list entries in jk[0] / bias[0], those of stage
    // s + 2 in jk[1]
    auto stage = [&](const int s, auto P) {
      // stage s has landed once at most the next stage's 16 loads are pending
      asm volatile("" ::: "memory");
      if (s + 1 < nst)
        __builtin_amdgcn_s_waitcnt((1 << 14) | (7 << 4) | (15 << 8));  // vmcnt(16)
      else
        __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0)
      asm volatile("" ::: "memory");
      const unsigned char* KT = sk[P()];
      const unsigned char* VT = sv[P()];
      // S^T = K Q^T: register i is key 8(i/4) + 4hi + i%4 of the stage
      dma::f32x16 sc;
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[i] = 0.f;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const dma::bf16x8 kop = *reinterpret_cast<const dma::bf16x8*>(
            KT + l32 * kDRowB + (((2 * kk + hi) ^ dswz(l32)) << 4));
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qf[kk], sc, 0, 0, 0);
      }
      // logits with the keys' bias, the stage's max and the new running max
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = 8 * (i >> 2) + 4 * hi + (i & 3);
        const float bk = __shfl(bias[0], 32 * P() + key);
        const float v = s * kStageKeys + key < nk ? fmaf(sc[i], a.scale, bk) : -INFINITY;
        sc[i] = v;
        mx = fmaxf(mx, v);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mn = fmaxf(m, mx);
      const float alpha = m == mn ? 1.f : __expf(m - mn);
      m = mn;
      dma::bf16x8 pb[2];
      float ls = 0.f, lrs = 0.f;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        float p[8];
#pragma unroll
        for (int t8 = 0; t8 < 8; ++t8) {
          p[t8] = __expf(sc[hf * 8 + t8] - mn);
          ls += p[t8];
        }
        pb[hf] = dma::to_bf16x8(p);
#pragma unroll
        for (int t8 = 0; t8 < 8; ++t8) lrs += (float)pb[hf][t8];
      }
      l = fmaf(l, alpha, ls);
      lr = fmaf(lr, alpha, lrs);
      if (dma::ballot(alpha != 1.f)) {  // some column's max grew
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
      }
      // O^T += V^T P^T over two 16-key steps; V read with the transposing load
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int k0r = 16 * hf + 4 * (g >> 1) + (r >> 2);
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
                                                          pb[hf], o[db], 0, 0, 0);
        }
      }
      // buffer P is free once its reads have returned: stage s+2 goes there
      if (s + 2 < nst) {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));  // lgkmcnt(0)
        asm volatile("" ::: "memory");
        issue(jk[1], P);
      }
    };
#pragma unroll 1
    for (int s = 0; s < nst; s += 2) {
      stage(s, P0{});
      if (s + 1 < nst) stage(s + 1, P1{});
      // the next pair's entries move to register 0
#pragma unroll
      for (int i = 0; i + 1 < kMaxStages / 2; ++i) {
        jk[i] = jk[i + 1];
        bias[i] = bias[i + 1];
      }
    }
    l += __shfl_xor(l, 32);
    lr += __shfl_xor(lr, 32);
  }
  // this wave's (max, sum, o) for query head n: register i of block db is
  // d = db*32 + 8(i/4) + 4hi + i%4.  o is stored as l/lr times the product, so
  // that o / l, what the merge divides by, is the product over lr.  FUSED: in
  // the wave's own LDS (its loads have all landed and been read), else in the
  // workspace
  float* part = FUSED ? reinterpret_cast<float*>(s_wave) + min(n, G - 1) * 130
                      : static_cast<float*>(a.ws) +
                            (((int64_t)b * a.Hq + h * G + min(n, G - 1)) * nsplit + split) * 130;
  if (n < G) {
    const float f = lr > 0.f ? l / lr : 0.f;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[db][i] *= f;
    if (hi == 0) {
      part[0] = m;
      part[1] = l;
    }
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
        for (int k = 0; k < 4; ++k) part[2 + db * 32 + 8 * q4 + 4 * hi + k] = o[db][4 * q4 + k];
  }
  if constexpr (FUSED) {
    // the merge of decode_combine_kernel over the workgroup's waves, in the
    // same order and arithmetic; one (query head, d) per thread
    __syncthreads();
    for (int t = threadIdx.x; t < G * 128; t += blockDim.x) {
      const int nn = t >> 7, d = t & 127;
      float M = -INFINITY;
      for (int sp = 0; sp < nsplit; ++sp)
        M = fmaxf(M, reinterpret_cast<const float*>(s_dyn + sp * 4 * kStageBytes)[nn * 130]);
      float L = 0.f, ov = 0.f;
      if (M != -INFINITY) {
        for (int sp = 0; sp < nsplit; ++sp) {
          const float* pp = reinterpret_cast<const float*>(s_dyn + sp * 4 * kStageBytes) + nn * 130;
          const float fs = expf(pp[0] - M);
          L = fmaf(pp[1], fs, L);
          ov = fmaf(pp[2 + d], fs, ov);
        }
      }
      const float res = L > 0.f ? ov / L : 0.f;
      const int hq = h * G + nn;
      static_cast<__bf16*>(a.O)[((int64_t)b * a.Sq * a.Hq + hq) * 128 + d] = (__bf16)res;
      if (a.lse && d == 0) a.lse[(int64_t)b * a.Hq + hq] = M + logf(L) + dmax;
    }
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

// Entries per wave: enough waves for whole rounds of the LDS-bound five per
// CU, at most 512 entries (16 stages) and at least 64 per wave.
int pipe_range(int64_t BH, int64_t u_stride) {
  const int64_t slots = (int64_t)dma_cu_count() * kPipeWavesPerCU;
  int64_t per = std::max<int64_t>((u_stride + kMaxStages * kStageKeys - 1) /
                                      (kMaxStages * kStageKeys),
                                  (slots + BH - 1) / BH);
  const int64_t rounds = (BH * per + slots - 1) / slots;
  per = std::max<int64_t>(per, rounds * slots / BH);
  per = std::min<int64_t>(per, (u_stride + kMinRange - 1) / kMinRange);
  int64_t range = (u_stride + per - 1) / per;
  range = (range + kStageKeys - 1) / kStageKeys * kStageKeys;
  return (int)std::max<int64_t>(range, kMinRange);
}

hipError_t launch_mfma(const DmaAttnArgs& a, hipStream_t st) {
  const int range = pipe_range(a.B * a.Hkv, a.u_stride);
  const int nsplit = (int)((a.u_stride + range - 1) / range);
  const size_t wave_lds = 4 * kStageBytes;
  if (nsplit == kPipeWavesPerCU) {
    // one workgroup per (batch, kv head) fills a CU's LDS: merge in place
    const void* fn = reinterpret_cast<const void*>(&decode_mfma_kernel<true>);
    (void)dma_func_max_lds(fn, nsplit * wave_lds);
    hipLaunchKernelGGL(decode_mfma_kernel<true>, dim3(1, (unsigned)a.Hkv, (unsigned)a.B),
                       dim3(64 * nsplit), nsplit * wave_lds, st, a, nsplit, range);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(decode_mfma_kernel<false>,
                     dim3((unsigned)nsplit, (unsigned)a.Hkv, (unsigned)a.B), dim3(64), wave_lds,
                     st, a, nsplit, range);
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
  // enough for either path: at least 64 entries per split (bf16, D = 128) or 256
  const int64_t nsplit = std::max<int64_t>((u_stride + kMinRange - 1) / kMinRange,
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
