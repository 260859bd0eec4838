// Dynamic weights of the DMA forward (Hugging Face blog "Trainable Dynamic
// Mask Sparse Attention", section "Dynamic Sparse Mask Generation", delta
// equation): delta[b,h,j] = exp(softplus(V[b,j,:] . Delta[:,h]) * A[h]).
//
// HBM-bound: every value row (Hkv*D elements) is read once with coalesced
// 16-byte loads; the weight matrix slice sits in LDS.  A workgroup of four
// waves handles 32 consecutive keys of one sequence; each wave takes 8 keys
// in two groups of 4 so that one LDS read of the weights feeds 4 rows.
#include "common.h"

namespace {

constexpr int kRowsPerBlock = 32;
constexpr int kRowsPerGroup = 4;

template <typename T>
struct Chunk;
template <>
struct Chunk<float> {
  static constexpr int kElems = 4;
  __device__ static float get(const uint4& r, int e) {
    const uint32_t w = e == 0 ? r.x : e == 1 ? r.y : e == 2 ? r.z : r.w;
    return __uint_as_float(w);
  }
};
template <>
struct Chunk<__bf16> {
  static constexpr int kElems = 8;
  __device__ static float get(const uint4& r, int e) {
    const uint32_t w = (e >> 1) == 0 ? r.x : (e >> 1) == 1 ? r.y : (e >> 1) == 2 ? r.z : r.w;
    return (e & 1) ? dma::bf16_hi(w) : dma::bf16_lo(w);
  }
};

// Sum each of the HB per-lane partials over the wave.  Halving exchanges hand
// half the values to the partner lane at each step, so lane l ends with the
// full sum of head `head` (each head is held by 64/HB lanes).
template <int HB, int N>
__device__ __forceinline__ void halve(float (&v)[HB], int lane, int o, int& head) {
  const bool up = (lane & o) != 0;
#pragma unroll
  for (int k = 0; k < N / 2; ++k) {
    const float send = up ? v[k] : v[k + N / 2];
    const float keep = up ? v[k + N / 2] : v[k];
    v[k] = keep + __shfl_xor(send, o);
  }
  if (up) head += N / 2;
}

template <int HB>
__device__ __forceinline__ float reduce_heads(float (&v)[HB], int lane, int& head) {
  head = 0;
  int o = 32;
  if constexpr (HB >= 8) { halve<HB, 8>(v, lane, o, head); o >>= 1; }
  if constexpr (HB >= 4) { halve<HB, 4>(v, lane, o, head); o >>= 1; }
  if constexpr (HB >= 2) { halve<HB, 2>(v, lane, o, head); o >>= 1; }
  for (; o >= 1; o >>= 1) v[0] += __shfl_xor(v[0], o);
  return v[0];
}

__device__ __forceinline__ float softplus_f(float x) {
  return x > 0.f ? x + log1pf(expf(-x)) : log1pf(expf(x));
}

template <typename T, int HB>
__global__ __launch_bounds__(256) void weights_kernel(const T* __restrict__ V, int64_t sb,
                                                      int64_t ss, int Sk, int C, int Hkv, int h0,
                                                      const float* __restrict__ Delta,
                                                      const float* __restrict__ A,
                                                      float* __restrict__ delta) {
  extern __shared__ float smem[];
  // Delta slice laid out [h][e][k] (c = k*EPC + e): lanes own consecutive chunks k,
  // so for a fixed (h, e) a wave reads 64 consecutive words, free of bank conflicts.
  constexpr int EPC = Chunk<T>::kElems;
  const int NC = C / EPC;
  float* Ds = smem;                 // [HB][EPC][NC]
  float* sout = smem + C * HB;      // [HB][kRowsPerBlock]
  const int b = blockIdx.y;
  const int j0 = blockIdx.x * kRowsPerBlock;
  // 8 loads per thread in flight at a time (clamped addresses, masked after)
  constexpr int kFill = 8;
  for (int i0 = threadIdx.x; i0 < C * HB; i0 += 256 * kFill) {
    float v[kFill];
#pragma unroll
    for (int u = 0; u < kFill; ++u) {
      const int i = min(i0 + u * 256, C * HB - 1);
      const int c = i / HB, h = i % HB;
      v[u] = Delta[(int64_t)c * Hkv + min(h0 + h, Hkv - 1)];
    }
#pragma unroll
    for (int u = 0; u < kFill; ++u) {
      const int i = i0 + u * 256;
      const int c = i / HB, h = i % HB;
      if (i < C * HB) Ds[(h * EPC + c % EPC) * NC + c / EPC] = (h0 + h < Hkv) ? v[u] : 0.f;
    }
  }
  __syncthreads();

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const T* Vb = V + (int64_t)b * sb;
  for (int g = 0; g < 2; ++g) {
    const int jb = j0 + wave * 8 + g * kRowsPerGroup;
    float acc[kRowsPerGroup][HB];
#pragma unroll
    for (int r = 0; r < kRowsPerGroup; ++r)
#pragma unroll
      for (int h = 0; h < HB; ++h) acc[r][h] = 0.f;
    for (int k = lane; k < NC; k += 64) {
      uint4 raw[kRowsPerGroup];
#pragma unroll
      for (int r = 0; r < kRowsPerGroup; ++r) {
        // rows past the end read the last row; their sums are not written
        const int j = min(jb + r, Sk - 1);
        raw[r] = *reinterpret_cast<const uint4*>(Vb + (int64_t)j * ss + k * EPC);
      }
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        float dh[HB];
#pragma unroll
        for (int h = 0; h < HB; ++h) dh[h] = Ds[(h * EPC + e) * NC + k];
#pragma unroll
        for (int r = 0; r < kRowsPerGroup; ++r) {
          const float x = Chunk<T>::get(raw[r], e);
#pragma unroll
          for (int h = 0; h < HB; ++h) acc[r][h] = fmaf(x, dh[h], acc[r][h]);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < kRowsPerGroup; ++r) {
      int head;
      const float pre = reduce_heads<HB>(acc[r], lane, head);
      if ((lane & (64 / HB - 1)) == 0) sout[head * kRowsPerBlock + wave * 8 + g * 4 + r] = pre;
    }
  }
  __syncthreads();
  for (int t = threadIdx.x; t < HB * kRowsPerBlock; t += blockDim.x) {
    const int h = t / kRowsPerBlock, jj = t % kRowsPerBlock;
    const int j = j0 + jj;
    if (j < Sk && h0 + h < Hkv) {
      const float sp = softplus_f(sout[t]);
      delta[((int64_t)b * Hkv + h0 + h) * Sk + j] = expf(sp * A[h0 + h]);
    }
  }
}

template <typename T, int HB>
hipError_t launch(const T* V, int64_t B, int64_t Sk, int64_t Hkv, int64_t D, int64_t sb,
                  int64_t ss, const float* Delta, const float* A, float* delta, hipStream_t st) {
  const int C = (int)(Hkv * D);
  const size_t lds = (size_t)(C * HB + HB * kRowsPerBlock) * sizeof(float);
  dim3 grid((unsigned)((Sk + kRowsPerBlock - 1) / kRowsPerBlock), (unsigned)B,
            (unsigned)((Hkv + HB - 1) / HB));
  for (int hz = 0; hz < (int)grid.z; ++hz) {
    dim3 g2(grid.x, grid.y, 1);
    hipLaunchKernelGGL((weights_kernel<T, HB>), g2, dim3(256), lds, st, V, sb, ss, (int)Sk, C,
                       (int)Hkv, hz * HB, Delta, A, delta);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const T* V, int64_t B, int64_t Sk, int64_t Hkv, int64_t D, int64_t sb,
                    int64_t ss, const float* Delta, const float* A, float* delta, hipStream_t st) {
  if (Hkv >= 8) return launch<T, 8>(V, B, Sk, Hkv, D, sb, ss, Delta, A, delta, st);
  if (Hkv >= 4) return launch<T, 4>(V, B, Sk, Hkv, D, sb, ss, Delta, A, delta, st);
  if (Hkv >= 2) return launch<T, 2>(V, B, Sk, Hkv, D, sb, ss, Delta, A, delta, st);
  return launch<T, 1>(V, B, Sk, Hkv, D, sb, ss, Delta, A, delta, st);
}

}  // namespace

hipError_t dma_launch_weights(const void* V, int is_bf16, int64_t B, int64_t Sk, int64_t Hkv,
                              int64_t D, int64_t sb, int64_t ss, const float* Delta,
                              const float* A, float* delta, hipStream_t st) {
  if (is_bf16)
    return launch_t<__bf16>(static_cast<const __bf16*>(V), B, Sk, Hkv, D, sb, ss, Delta, A, delta,
                            st);
  return launch_t<float>(static_cast<const float*>(V), B, Sk, Hkv, D, sb, ss, Delta, A, delta, st);
}
