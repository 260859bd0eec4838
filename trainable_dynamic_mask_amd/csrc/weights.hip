// Dynamic weights of the DMA forward (Hugging Face blog "Trainable Dynamic
// Mask Sparse Attention", section "Dynamic Sparse Mask Generation", delta
// equation): delta[b,h,j] = exp(softplus(V[b,j,:] . Delta[:,h]) * A[h]).
//
// HBM-bound: every value row (Hkv*D elements) is read once.
// - bf16 values: the contraction runs on the matrix cores.  Each fp32 weight
//   is split into three bf16 parts hi + mid + lo that sum to it exactly (each
//   residual has at most 16, then 8, significant bits), so the products are
//   exact and only the fp32 accumulation rounds.  The split weight slice sits
//   in LDS; each workgroup loads it once and then walks tiles of 32 keys in a
//   grid-stride loop, loading the next tile while the current one computes.
// - fp32 values: a vector-ALU kernel; a workgroup of four waves handles 32
//   consecutive keys, each wave 8 keys in two groups of 4 so that one LDS read
//   of the weights feeds 4 rows.
#include "common.h"

#include <algorithm>

namespace {

constexpr int kRowsPerBlock = 32;
constexpr int kRowsPerGroup = 4;

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

template <int HB>
__global__ __launch_bounds__(256) void weights_f32_kernel(const float* __restrict__ V, int64_t sb,
                                                      int64_t ss, int Sk, int C, int Hkv, int h0,
                                                      const float* __restrict__ Delta,
                                                      const float* __restrict__ A,
                                                      float* __restrict__ delta) {
  extern __shared__ float smem[];
  // Delta slice laid out [h][e][k] (c = k*EPC + e): lanes own consecutive chunks k,
  // so for a fixed (h, e) a wave reads 64 consecutive words, free of bank conflicts.
  constexpr int EPC = 4;   // fp32 values per 16-byte chunk
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
  const float* Vb = V + (int64_t)b * sb;
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
          const float x = __uint_as_float(e == 0 ? raw[r].x : e == 1 ? raw[r].y : e == 2 ? raw[r].z : raw[r].w);
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

// ---------------------------------------------------------------- bf16 values: MFMA
// x^T = Ds^T V^T on v_mfma_f32_32x32x16_bf16.  N = 32 keys of one tile; M =
// 24 used rows of the split weights (rows 0-7: hi of heads h0..h0+7, 8-15: mid,
// 16-23: lo; rows 24-31 read a zero row).  In the accumulator layout a lane
// (key n = lane%32, half = lane/32) holds hi, mid and lo of heads 4*half..+3
// for its key, so each head's sum is formed without exchanging lanes.  The
// 16-channel k-steps are shared out among the W waves (contiguous ranges);
// their partial sums meet in LDS.  At k-step s, lane half hh reads channel
// chunk 2s+hh (8 channels), so the two lanes of a key read 32 contiguous bytes
// of its row and a wave walks a contiguous range of every row of the tile.
constexpr int kKeysPerTile = 32;
constexpr int kSplitRows = 25;  // 8 heads x {hi, mid, lo}, then one zero row
constexpr int kRedRows = 12;    // accumulator entries a lane contributes (rows 0..23)

__device__ __forceinline__ void split3(float d, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  hi = dma::f32_to_bf16_bits(d);
  const float r1 = d - __uint_as_float(hi << 16);   // exact
  mid = dma::f32_to_bf16_bits(r1);
  const float r2 = r1 - __uint_as_float(mid << 16);  // exact, at most 8 significant bits
  lo = dma::f32_to_bf16_bits(r2);
}

// BWD: instead of delta, the epilogue forms the gradient of the
// pre-activation from ddelta = dL/ddelta (its load travels with the tile's
// values): dpre[b,j,h] = ddelta * delta * A[h] * sigmoid(pre), and adds
// ddelta * delta * softplus(pre) over the tile's keys into dA[h].
template <int W, int NS, bool BWD>
__global__ __launch_bounds__(64 * W, 2) void weights_mfma_kernel(
    const __bf16* __restrict__ V, int64_t sb, int64_t ss, int Sk, int B, int C, int Hkv, int h0,
    const float* __restrict__ Delta, const float* __restrict__ A, float* __restrict__ delta,
    const float* __restrict__ ddelta, float* __restrict__ dpre, float* __restrict__ dA) {
  extern __shared__ __align__(16) unsigned char smem_m[];
  const int nchunks = C / 8;
  uint4* ds = reinterpret_cast<uint4*>(smem_m);        // [C/8][25] chunks of 8 bf16
  float* red = reinterpret_cast<float*>(smem_m + (size_t)nchunks * kSplitRows * 16);  // [2][W][12][64]
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int n = lane & 31, hh = lane >> 5;
  const int nsteps = C / 16;
  const int per = (nsteps + W - 1) / W;
  const int s0 = min(nsteps, wave * per);
  const int ns = min(nsteps, s0 + per) - s0;  // k-steps of this wave (uniform)
  const int tps = (Sk + kKeysPerTile - 1) / kKeysPerTile;
  const int ntiles = B * tps;

  // every load is issued (steps past this wave's range repeat its last chunk,
  // keys past the end repeat the last key), so the load count never branches
  // the epilogue thread (key nn, head h) of this thread's index
  const int e_nn = threadIdx.x % kKeysPerTile, e_h = min((int)threadIdx.x / kKeysPerTile, 7);
  auto issue = [&](uint4 (&buf)[NS], float& gd, int t) {
    const int b = t / tps;
    const int j = min((t - b * tps) * kKeysPerTile + n, Sk - 1);
    const __bf16* row = V + (int64_t)b * sb + (int64_t)j * ss;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int kc = 2 * max(0, min(s0 + min(s, ns - 1), nsteps - 1)) + hh;
      buf[s] = *reinterpret_cast<const uint4*>(row + kc * 8);
    }
    if constexpr (BWD) {
      const int je = min((t - b * tps) * kKeysPerTile + e_nn, Sk - 1);
      gd = ddelta[((int64_t)b * Hkv + min(h0 + e_h, Hkv - 1)) * Sk + je];
    }
  };

  // the epilogue thread (key nn, head h) needs A[h0+h]: loaded once, up front,
  // since a load inside the loop would also wait for the prefetched tile
  const float a_h = A[min(h0 + (int)(threadIdx.x / kKeysPerTile) % 8, Hkv - 1)];

  auto consume = [&](const uint4 (&buf)[NS], float gd, int t, float* rb) {
    dma::f32x16 acc = {};
    const uint4* arow = ds + (2 * s0 + hh) * kSplitRows + min(n, kSplitRows - 1);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (s < ns) {
        const uint4 a = arow[s * 2 * kSplitRows];
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(dma::bf16x8, a),
                                                      __builtin_bit_cast(dma::bf16x8, buf[s]),
                                                      acc, 0, 0, 0);
      }
    }
    float* my = rb + wave * kRedRows * 64;
#pragma unroll
    for (int i = 0; i < kRedRows; ++i) my[i * 64 + lane] = acc[i];
    __syncthreads();
    if (threadIdx.x < 8 * kKeysPerTile) {
      const int nn = threadIdx.x % kKeysPerTile, h = threadIdx.x / kKeysPerTile;
      const int l = nn + 32 * (h >> 2), i = h & 3;
      float xh = 0.f, xm = 0.f, xl = 0.f;
#pragma unroll
      for (int w = 0; w < W; ++w) {
        xh += rb[(w * kRedRows + i) * 64 + l];
        xm += rb[(w * kRedRows + i + 4) * 64 + l];
        xl += rb[(w * kRedRows + i + 8) * 64 + l];
      }
      const float x = xh + (xm + xl);
      const int b = t / tps;
      const int j = (t - b * tps) * kKeysPerTile + nn;
      const bool valid = j < Sk && h0 + h < Hkv;
      if constexpr (!BWD) {
        if (valid) delta[((int64_t)b * Hkv + h0 + h) * Sk + j] = expf(softplus_f(x) * a_h);
      } else {
        const float sp = softplus_f(x);
        const float dl = expf(sp * a_h);
        const float sig = 1.f / (1.f + expf(-x));
        if (valid) dpre[((int64_t)b * Sk + j) * Hkv + h0 + h] = gd * dl * a_h * sig;
        // dA[h]: sum over the tile's 32 keys (one 32-lane half of a wave)
        float g = valid ? gd * dl * sp : 0.f;
#pragma unroll
        for (int o = 16; o >= 1; o >>= 1) g += __shfl_xor(g, o);
        if (nn == 0 && h0 + h < Hkv) atomicAdd(&dA[h0 + h], g);
      }
    }
  };

  // split weight slice.  Slot q = (chunk kc, head h) holds channels 8kc..8kc+7
  // of head h0+h; it lands in rows h, 8+h, 16+h of chunk kc.  Its loads are
  // issued before the first tile's values so that waiting for them does not
  // wait for the tile (load counters retire in order).
  constexpr int kSlots = 4;  // C <= 256 * W slots per workgroup of W waves
  float d[kSlots][8];
#pragma unroll
  for (int u = 0; u < kSlots; ++u) {
    const int q = min(u * 64 * W + (int)threadIdx.x, C - 1);
    const int kc = q >> 3, h = q & 7;
#pragma unroll
    for (int e = 0; e < 8; ++e) d[u][e] = Delta[(int64_t)(kc * 8 + e) * Hkv + min(h0 + h, Hkv - 1)];
  }
  uint4 b0[NS], b1[NS];
  float g0 = 0.f, g1 = 0.f;
  int t = blockIdx.x;  // the grid never exceeds the tile count
  issue(b0, g0, t);
#pragma unroll
  for (int u = 0; u < kSlots; ++u) {
    const int q = u * 64 * W + (int)threadIdx.x;
    if (q < C) {
      const int kc = q >> 3, h = q & 7;
      uint32_t hi[8], mid[8], lo[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) split3(h0 + h < Hkv ? d[u][e] : 0.f, hi[e], mid[e], lo[e]);
      ds[kc * kSplitRows + h] = make_uint4(hi[0] | hi[1] << 16, hi[2] | hi[3] << 16,
                                           hi[4] | hi[5] << 16, hi[6] | hi[7] << 16);
      ds[kc * kSplitRows + 8 + h] = make_uint4(mid[0] | mid[1] << 16, mid[2] | mid[3] << 16,
                                               mid[4] | mid[5] << 16, mid[6] | mid[7] << 16);
      ds[kc * kSplitRows + 16 + h] = make_uint4(lo[0] | lo[1] << 16, lo[2] | lo[3] << 16,
                                                lo[4] | lo[5] << 16, lo[6] | lo[7] << 16);
    }
  }
  for (int kc = threadIdx.x; kc < nchunks; kc += 64 * W)
    ds[kc * kSplitRows + kSplitRows - 1] = make_uint4(0, 0, 0, 0);
  __syncthreads();

  // each path issues its prefetch unconditionally, so the compiler's load
  // counters stay exact and a tile's wait never covers the next tile's loads
  float* red0 = red;
  float* red1 = red + W * kRedRows * 64;
  while (true) {
    const int t1 = t + gridDim.x;
    if (t1 >= ntiles) {
      consume(b0, g0, t, red0);
      break;
    }
    issue(b1, g1, t1);
    consume(b0, g0, t, red0);
    const int t2 = t1 + gridDim.x;
    if (t2 >= ntiles) {
      consume(b1, g1, t1, red1);
      break;
    }
    issue(b0, g0, t2);
    consume(b1, g1, t1, red1);
    t = t2;
  }
}

// Backward of the contraction, given dpre [B,Sk,Hkv]: one workgroup per
// (batch, 256 keys, 256 channels), one channel per thread, eight heads at a
// time, eight keys per step so that their loads are in flight together:
//   dV[b,j,c]   += sum_h dpre[b,j,h] Delta[c,h]     (added to the attention's dV)
//   dDelta[c,h] += sum_j V[b,j,c] dpre[b,j,h]       (per-workgroup sums, then atomics)
constexpr int kBwdKeys = 256;

__global__ __launch_bounds__(256) void weights_bwd_kernel(const __bf16* __restrict__ V, int64_t sb,
                                                          int64_t ss, int Sk, int C, int Hkv,
                                                          const float* __restrict__ Delta,
                                                          const float* __restrict__ dpre,
                                                          float* __restrict__ dV,
                                                          float* __restrict__ dDelta) {
  __shared__ float s_p[kBwdKeys][8];
  const int b = blockIdx.z, jb = blockIdx.x * kBwdKeys, tid = threadIdx.x;
  const int c = blockIdx.y * 256 + tid;
  const int cc = min(c, C - 1);
  const int nj = min(kBwdKeys, Sk - jb);
  const __bf16* Vb = V + (int64_t)b * sb + (int64_t)jb * ss + cc;
  float* dVb = dV + ((int64_t)b * Sk + jb) * C + cc;
  for (int h0 = 0; h0 < Hkv; h0 += 8) {
    float dD[8], Dl[8];
#pragma unroll
    for (int h = 0; h < 8; ++h) {
      dD[h] = 0.f;
      Dl[h] = h0 + h < Hkv ? Delta[(int64_t)cc * Hkv + h0 + h] : 0.f;
    }
    __syncthreads();
    for (int e = tid; e < kBwdKeys * 8; e += 256) {
      const int jj = e >> 3, h = e & 7;
      s_p[jj][h] = (jj < nj && h0 + h < Hkv) ? dpre[((int64_t)b * Sk + jb + jj) * Hkv + h0 + h]
                                             : 0.f;
    }
    __syncthreads();
    for (int j8 = 0; j8 < nj; j8 += 8) {
      float v[8], o[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int jj = min(j8 + u, nj - 1);
        v[u] = (float)Vb[(int64_t)jj * ss];
        o[u] = dVb[(int64_t)jj * C];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int jj = j8 + u;
        if (jj < nj) {
          float acc = 0.f;
#pragma unroll
          for (int h = 0; h < 8; ++h) {
            const float p = s_p[jj][h];
            dD[h] = fmaf(v[u], p, dD[h]);
            acc = fmaf(p, Dl[h], acc);
          }
          if (c < C) dVb[(int64_t)jj * C] = o[u] + acc;
        }
      }
    }
    if (c < C)
#pragma unroll
      for (int h = 0; h < 8; ++h)
        if (h0 + h < Hkv) atomicAdd(&dDelta[(int64_t)c * Hkv + h0 + h], dD[h]);
  }
}

__global__ void fill_zero_kernel(float* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0.f;
}

template <int W, int NS, bool BWD = false>
hipError_t launch_mfma(const __bf16* V, int64_t B, int64_t Sk, int64_t Hkv, int64_t D, int64_t sb,
                       int64_t ss, const float* Delta, const float* A, float* delta,
                       hipStream_t st, const float* ddelta = nullptr, float* dpre = nullptr,
                       float* dA = nullptr) {
  const int C = (int)(Hkv * D);
  const size_t lds = (size_t)C / 8 * kSplitRows * 16 + (size_t)2 * W * kRedRows * 64 * 4;
  const int64_t ntiles = B * ((Sk + kKeysPerTile - 1) / kKeysPerTile);
  const int per_cu = std::max<int>(1, (int)((160 * 1024) / lds));
  const int64_t grid = std::min<int64_t>(ntiles, (int64_t)dma_cu_count() * per_cu);
  (void)dma_func_max_lds(reinterpret_cast<const void*>(&weights_mfma_kernel<W, NS, BWD>), lds);
  for (int h0 = 0; h0 < Hkv; h0 += 8)
    hipLaunchKernelGGL((weights_mfma_kernel<W, NS, BWD>), dim3((unsigned)grid), dim3(64 * W), lds,
                       st, V, sb, ss, (int)Sk, (int)B, C, (int)Hkv, h0, Delta, A, delta, ddelta,
                       dpre, dA);
  return hipGetLastError();
}

// k-steps of 16 channels: C/16 = Hkv*D/16 <= 128; four waves share them up to
// C = 1024, eight above, so that no wave takes more than 16.
hipError_t launch_bf16_bwd(const __bf16* V, int64_t B, int64_t Sk, int64_t Hkv, int64_t D,
                           int64_t sb, int64_t ss, const float* Delta, const float* A,
                           const float* ddelta, float* dpre, float* dA, hipStream_t st) {
  const int64_t nsteps = Hkv * D / 16;
  if (nsteps > 64)
    return launch_mfma<8, 16, true>(V, B, Sk, Hkv, D, sb, ss, Delta, A, nullptr, st, ddelta, dpre, dA);
  const int64_t per = (nsteps + 3) / 4;
  if (per > 8)
    return launch_mfma<4, 16, true>(V, B, Sk, Hkv, D, sb, ss, Delta, A, nullptr, st, ddelta, dpre, dA);
  if (per > 4)
    return launch_mfma<4, 8, true>(V, B, Sk, Hkv, D, sb, ss, Delta, A, nullptr, st, ddelta, dpre, dA);
  return launch_mfma<4, 4, true>(V, B, Sk, Hkv, D, sb, ss, Delta, A, nullptr, st, ddelta, dpre, dA);
}

hipError_t launch_bf16(const __bf16* V, int64_t B, int64_t Sk, int64_t Hkv, int64_t D, int64_t sb,
                       int64_t ss, const float* Delta, const float* A, float* delta,
                       hipStream_t st) {
  const int64_t nsteps = Hkv * D / 16;
  if (nsteps > 64) return launch_mfma<8, 16>(V, B, Sk, Hkv, D, sb, ss, Delta, A, delta, st);
  const int64_t per = (nsteps + 3) / 4;
  if (per > 8) return launch_mfma<4, 16>(V, B, Sk, Hkv, D, sb, ss, Delta, A, delta, st);
  if (per > 4) return launch_mfma<4, 8>(V, B, Sk, Hkv, D, sb, ss, Delta, A, delta, st);
  return launch_mfma<4, 4>(V, B, Sk, Hkv, D, sb, ss, Delta, A, delta, st);
}

// ---------------------------------------------------------------- fp32 values
template <int HB>
hipError_t launch_f32(const float* V, int64_t B, int64_t Sk, int64_t Hkv, int64_t D, int64_t sb,
                      int64_t ss, const float* Delta, const float* A, float* delta,
                      hipStream_t st) {
  const int C = (int)(Hkv * D);
  const size_t lds = (size_t)(C * HB + HB * kRowsPerBlock) * sizeof(float);
  dim3 grid((unsigned)((Sk + kRowsPerBlock - 1) / kRowsPerBlock), (unsigned)B, 1);
  for (int h0 = 0; h0 < Hkv; h0 += HB)
    hipLaunchKernelGGL((weights_f32_kernel<HB>), grid, dim3(256), lds, st, V, sb, ss, (int)Sk, C,
                       (int)Hkv, h0, Delta, A, delta);
  return hipGetLastError();
}

hipError_t launch_f32_t(const float* V, int64_t B, int64_t Sk, int64_t Hkv, int64_t D, int64_t sb,
                        int64_t ss, const float* Delta, const float* A, float* delta,
                        hipStream_t st) {
  if (Hkv >= 8) return launch_f32<8>(V, B, Sk, Hkv, D, sb, ss, Delta, A, delta, st);
  if (Hkv >= 4) return launch_f32<4>(V, B, Sk, Hkv, D, sb, ss, Delta, A, delta, st);
  if (Hkv >= 2) return launch_f32<2>(V, B, Sk, Hkv, D, sb, ss, Delta, A, delta, st);
  return launch_f32<1>(V, B, Sk, Hkv, D, sb, ss, Delta, A, delta, st);
}

}  // namespace

hipError_t dma_launch_fill_zero(float* p, int64_t n, hipStream_t st) {
  hipLaunchKernelGGL(fill_zero_kernel, dim3(64), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

hipError_t dma_launch_weights_bwd(const void* V, int64_t B, int64_t Sk, int64_t Hkv, int64_t D,
                                  int64_t sb, int64_t ss, const float* Delta, const float* A,
                                  const float* ddelta, float* dV, float* dDelta, float* dA,
                                  float* dpre, hipStream_t st) {
  const int C = (int)(Hkv * D);
  hipLaunchKernelGGL(fill_zero_kernel, dim3(64), dim3(256), 0, st, dDelta, (int64_t)C * Hkv);
  hipLaunchKernelGGL(fill_zero_kernel, dim3(1), dim3(256), 0, st, dA, Hkv);
  const __bf16* Vb = static_cast<const __bf16*>(V);
  hipError_t e = launch_bf16_bwd(Vb, B, Sk, Hkv, D, sb, ss, Delta, A, ddelta, dpre, dA, st);
  if (e != hipSuccess) return e;
  dim3 grid((unsigned)((Sk + kBwdKeys - 1) / kBwdKeys), (unsigned)((C + 255) / 256), (unsigned)B);
  hipLaunchKernelGGL(weights_bwd_kernel, grid, dim3(256), 0, st, Vb, sb, ss, (int)Sk, C, (int)Hkv,
                     Delta, dpre, dV, dDelta);
  return hipGetLastError();
}

hipError_t dma_launch_weights(const void* V, int is_bf16, int64_t B, int64_t Sk, int64_t Hkv,
                              int64_t D, int64_t sb, int64_t ss, const float* Delta,
                              const float* A, float* delta, hipStream_t st) {
  if (is_bf16)
    return launch_bf16(static_cast<const __bf16*>(V), B, Sk, Hkv, D, sb, ss, Delta, A, delta, st);
  return launch_f32_t(static_cast<const float*>(V), B, Sk, Hkv, D, sb, ss, Delta, A, delta, st);
}
