// Masked attention of the DMA forward for fp32 inputs (Hugging Face blog
// "Trainable Dynamic Mask Sparse Attention", section "Efficient Sparse
// Attention Computation"), computed in fp32 throughout.  Same work split as
// the bf16 path: a workgroup takes one 64-row query tile of one kv head and
// walks the compacted key list of that tile in chunks of 64 gathered keys;
// its waves are query heads of the kv head.  Here each lane owns one query
// row, so the softmax needs no cross-lane reductions; keys are read from LDS
// as broadcasts.  This path favours exactness over speed: the bias is taken
// relative to the largest delta among the row's own kept keys (found by a
// first pass over the list), so delta - reference is exact for every key
// within a factor 2 of it, whatever the range of delta across the tile.
#include "common.h"

namespace {

constexpr int kBq = 64;
constexpr int kBk = 64;

template <int D>
struct SmemF {
  float k[kBk][D];
  float v[kBk][D];
  int pj[kBk];
  int e[kBk];
  float dlt[kBk];   // delta of the key, -inf for padding
};

template <int D, int NH>
__global__ __launch_bounds__(NH * 64, 1) void attn_prefill_f32_kernel(DmaAttnArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  SmemF<D>& sm = *reinterpret_cast<SmemF<D>*>(smem_raw);
  constexpr int NT = NH * 64;
  // keys per online-softmax update (4 with D = 128: q and o take 256 registers)
  constexpr int kGroup = D == 128 ? 4 : 8;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = (int)(a.Hq / a.Hkv);
  const int ngrp = G / NH;
  const int t = blockIdx.x, h = blockIdx.y;
  const int b = blockIdx.z / ngrp, hgrp = blockIdx.z % ngrp;
  const int hq = h * G + hgrp * NH + wave;
  const int64_t seg = (int64_t)b * a.Hkv + h;
  const int64_t g = seg * a.n_tiles + t;
  const int r_lo = t * kBq;
  const int rows = min(kBq, (int)a.Sq - r_lo);
  const int pos = (int)a.q0 + r_lo + lane;
  const int cnt = a.u_cnt[g];
  const int32_t* list = a.u_idx + g * a.u_stride;
  const float* dl = a.delta + seg * a.Sk;
  const int32_t* ev = a.evict + seg * a.Sk;
  const float* Kg = static_cast<const float*>(a.K) + b * a.ksb + h * a.ksh;
  const float* Vg = static_cast<const float*>(a.V) + b * a.ksb + h * a.ksh;

  // the row's reference: the largest delta among its kept keys
  float rmax = -INFINITY;
  for (int c0 = 0; c0 < cnt; c0 += kBk) {
    __syncthreads();
    for (int kk = tid; kk < kBk; kk += NT) {
      const int idx = c0 + kk;
      const bool pad = idx >= cnt;
      const int j = pad ? 0 : list[idx];
      sm.pj[kk] = pad ? 0x7fffffff : j;
      sm.e[kk] = pad ? 0 : ev[j];
      sm.dlt[kk] = pad ? -INFINITY : dl[j];
    }
    __syncthreads();
    const int nk = min(kBk, cnt - c0);
    for (int kk = 0; kk < nk; ++kk)
      if (sm.pj[kk] <= pos && pos < sm.e[kk]) rmax = fmaxf(rmax, sm.dlt[kk]);
  }
  float q[D], o[D];
  {
    const float* qrow = static_cast<const float*>(a.Q) + b * a.qsb + hq * a.qsh +
                        (int64_t)(r_lo + (lane < rows ? lane : 0)) * a.qss;
#pragma unroll
    for (int d = 0; d < D; d += 4) {
      const float4 v = *reinterpret_cast<const float4*>(qrow + d);
      q[d] = v.x;
      q[d + 1] = v.y;
      q[d + 2] = v.z;
      q[d + 3] = v.w;
    }
#pragma unroll
    for (int d = 0; d < D; ++d) o[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;

  for (int c0 = 0; c0 < cnt; c0 += kBk) {
    __syncthreads();
    // stage the chunk: D/4 float4 per key row for K and V
    for (int u = tid; u < kBk * (D / 4); u += NT) {
      const int kk = u / (D / 4), ch = u % (D / 4);
      const int idx = c0 + kk;
      const int j = idx < cnt ? list[idx] : 0;
      *reinterpret_cast<float4*>(&sm.k[kk][ch * 4]) =
          *reinterpret_cast<const float4*>(Kg + (int64_t)j * a.kss + ch * 4);
      *reinterpret_cast<float4*>(&sm.v[kk][ch * 4]) =
          *reinterpret_cast<const float4*>(Vg + (int64_t)j * a.kss + ch * 4);
    }
    for (int kk = tid; kk < kBk; kk += NT) {
      const int idx = c0 + kk;
      const bool pad = idx >= cnt;
      const int j = pad ? 0 : list[idx];
      sm.pj[kk] = pad ? 0x7fffffff : j;
      sm.e[kk] = pad ? 0 : ev[j];
      sm.dlt[kk] = pad ? -INFINITY : dl[j];
    }
    __syncthreads();
    const int nk = min(kBk, cnt - c0);
    for (int k0 = 0; k0 < nk; k0 += kGroup) {
      float x[kGroup];
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < kGroup; ++r) {
        const int kk = k0 + r;
        float dot = 0.f;
#pragma unroll
        for (int d = 0; d < D; d += 4) {
          const float4 kv = *reinterpret_cast<const float4*>(&sm.k[kk][d]);
          dot = fmaf(q[d], kv.x, dot);
          dot = fmaf(q[d + 1], kv.y, dot);
          dot = fmaf(q[d + 2], kv.z, dot);
          dot = fmaf(q[d + 3], kv.w, dot);
        }
        const bool keep = kk < nk && sm.pj[kk] <= pos && pos < sm.e[kk];
        x[r] = keep ? fmaf(dot, a.scale, sm.dlt[kk] - rmax) : -INFINITY;
        mx = fmaxf(mx, x[r]);
      }
      const float m_new = fmaxf(m, mx);
      if (m_new == -INFINITY) continue;  // nothing kept yet for this row
      const float alpha = expf(m - m_new);
      float p[kGroup];
      float ps = 0.f;
#pragma unroll
      for (int r = 0; r < kGroup; ++r) {
        p[r] = expf(x[r] - m_new);
        ps += p[r];
      }
      l = l * alpha + ps;
      m = m_new;
#pragma unroll
      for (int d = 0; d < D; d += 4) {
        float4 acc = make_float4(o[d] * alpha, o[d + 1] * alpha, o[d + 2] * alpha, o[d + 3] * alpha);
#pragma unroll
        for (int r = 0; r < kGroup; ++r) {
          const float4 vv = *reinterpret_cast<const float4*>(&sm.v[k0 + r][d]);
          acc.x = fmaf(p[r], vv.x, acc.x);
          acc.y = fmaf(p[r], vv.y, acc.y);
          acc.z = fmaf(p[r], vv.z, acc.z);
          acc.w = fmaf(p[r], vv.w, acc.w);
        }
        o[d] = acc.x;
        o[d + 1] = acc.y;
        o[d + 2] = acc.z;
        o[d + 3] = acc.w;
      }
    }
  }

  if (lane < rows) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float* orow = static_cast<float*>(a.O) + (((int64_t)b * a.Sq + r_lo + lane) * a.Hq + hq) * D;
#pragma unroll
    for (int d = 0; d < D; d += 4)
      *reinterpret_cast<float4*>(orow + d) =
          make_float4(o[d] * inv, o[d + 1] * inv, o[d + 2] * inv, o[d + 3] * inv);
    if (a.lse) a.lse[((int64_t)b * a.Hq + hq) * a.Sq + r_lo + lane] = m + logf(l) + rmax;
  }
}

template <int D, int NH>
hipError_t launch(const DmaAttnArgs& a, hipStream_t st) {
  const int G = (int)(a.Hq / a.Hkv);
  dim3 grid((unsigned)a.n_tiles, (unsigned)a.Hkv, (unsigned)(a.B * (G / NH)));
  const size_t lds = sizeof(SmemF<D>);
  (void)dma_func_max_lds(reinterpret_cast<const void*>(&attn_prefill_f32_kernel<D, NH>), lds);
  hipLaunchKernelGGL((attn_prefill_f32_kernel<D, NH>), grid, dim3(NH * 64), lds, st, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DmaAttnArgs& a, hipStream_t st) {
  const int G = (int)(a.Hq / a.Hkv);
  if (G % 4 == 0) return launch<D, 4>(a, st);
  if (G % 2 == 0) return launch<D, 2>(a, st);
  return launch<D, 1>(a, st);
}

}  // namespace

hipError_t dma_launch_attn_prefill_f32(const DmaAttnArgs& a, hipStream_t st) {
  return a.D == 64 ? launch_d<64>(a, st) : launch_d<128>(a, st);
}
