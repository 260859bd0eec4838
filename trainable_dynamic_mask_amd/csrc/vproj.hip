// Value projection with the dynamic weights formed in its epilogue (Hugging
// Face blog "Trainable Dynamic Mask Sparse Attention", section "Dynamic
// Sparse Mask Generation": delta is computed from the value matrix, delta =
// exp(softplus(V Delta) * A)).
//
//   V[m, n]      = sum_k X[m, k] * Wv[k, n]        (m = b*Sk + j, fp32 accumulation,
//                                                    stored as bf16)
//   pre[m, h]    = sum_n Vbf16[m, n] * Delta[n, h]  (the stored values, as dma_weights
//                                                    reads them)
//   delta[b,h,j] = exp(softplus(pre[m, h]) * A[h])
//
// One workgroup of 8 waves computes a 256 x 256 tile of V on
// v_mfma_f32_32x32x16_bf16 (wave (wm, wn): rows 64*wm.., columns 128*wn..),
// K in steps of 64 through two LDS stages filled by direct 16-byte loads
// (the next stage in flight while the current one is multiplied, one barrier
// per step).  X rows are read as the A operand straight from LDS; Wv rows
// (k-major) become the B operand through the transposing LDS read.  The
// epilogue rounds the wave's 64 x 128 block to bf16 in LDS, stores it to V
// with whole-row 16-byte stores and, for the weights, multiplies it by the
// wave's 128 x 8 slice of Delta split into three bf16 parts that sum to it
// exactly (hi + mid + lo: the products are exact, only the fp32 sums round).
// The workgroup adds its two 128-column partial sums of pre through LDS; a
// second kernel adds the N/256 partials of each (key, head) in a fixed order
// and applies exp(softplus(.) * A), so the result does not depend on
// scheduling.
#include "lds_dma.h"

#include <algorithm>

namespace {

constexpr int kTileM = 256, kTileN = 256, kStepK = 64;
constexpr int kWaves = 8;
constexpr int kABytes = kTileM * kStepK * 2;         // 32 KB: X rows, 128 B each
constexpr int kBBytes = kStepK * kTileN * 2;         // 32 KB: two halves of 64 x 128
constexpr int kStageBytes = kABytes + kBBytes;
constexpr int kDsplitBytes = 32 * kTileN * 2;        // 16 KB: [32 rows][256 n] bf16
constexpr int kLdsBytes = 2 * kStageBytes + kDsplitBytes;
constexpr int kHeads = 8;                            // heads per fused epilogue

// chunk c of row r at c ^ (((r & 3) << 2) | ((r >> 2) & 3)) in 256-byte rows:
// conflict-free for the transposing reads
__device__ __forceinline__ int swz16(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

template <bool EPI>
__global__ __launch_bounds__(kWaves * 64, 1) void vproj_kernel(
    const __bf16* __restrict__ X, int64_t x_sb, int64_t x_ss, const __bf16* __restrict__ Wv,
    __bf16* __restrict__ V, int64_t v_sb, int64_t v_ss, int64_t M, int Sk, int Cin, int N,
    const float* __restrict__ Delta, int Hkv, float* __restrict__ pre_part, int nm_tiles) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int wm = wave & 3, wn = wave >> 2;
  const int l32 = lane & 31, hi = lane >> 5;
  // XCD-aware tile order: the N/256 column tiles of one row tile are
  // consecutive blocks of one XCD (blocks go round-robin over 8 XCDs), so
  // they share the X rows in that XCD's L2
  const int nn_tiles = N / kTileN;
  const int L = blockIdx.x;
  const int q = L >> 3;
  const int mt = (q / nn_tiles) * 8 + (L & 7), nt = q % nn_tiles;
  if (mt >= nm_tiles) return;
  const int64_t m0 = (int64_t)mt * kTileM;
  const int n0 = nt * kTileN;
  const uint32_t lds0 = dma::lds_addr(smem);
  unsigned char* const Ds = smem + 2 * kStageBytes;  // Delta's parts for the epilogue
  if constexpr (EPI) {
    // Delta's 256 x 8 slice of this column tile split into bf16 parts,
    // D3[s*8 + h][n] (s = hi, mid, lo; zero past Hkv heads and in rows
    // 24..31): [32 rows][256 n], 512-byte rows, 16-byte chunk c of row r at
    // c ^ r.  Thread t: column t/2, heads 4(t%2)..
    const int n = threadIdx.x >> 1, h0 = 4 * (threadIdx.x & 1);
    auto put = [&](int row, int col, __bf16 v) {
      *reinterpret_cast<__bf16*>(Ds + row * 512 + (((col >> 3) ^ row) << 4) + (col & 7) * 2) = v;
    };
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int h = h0 + t;
      const float d = h < Hkv ? Delta[(int64_t)(n0 + n) * Hkv + h] : 0.f;
      const __bf16 p0 = (__bf16)d;
      const float r1 = d - (float)p0;
      const __bf16 p1 = (__bf16)r1;
      put(h, n, p0);
      put(8 + h, n, p1);
      put(16 + h, n, (__bf16)(r1 - (float)p1));
      put(24 + h, n, (__bf16)0.f);
    }
  }

  // loads of one stage: wave w fills X rows 32w.. (4 pieces of 8 rows) and
  // Wv half w>>2, k rows 16(w&3).. (4 pieces of 4 rows)
  const __bf16* xrow[4];
  int xslot[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int r = 32 * wave + 8 * p + (lane >> 3);  // row of the tile
    const int64_t m = std::min<int64_t>(m0 + r, M - 1);  // rows past M repeat the last
    const int64_t b = m / Sk, j = m - b * Sk;
    xrow[p] = X + b * x_sb + j * x_ss;
    xslot[p] = (lane & 7) ^ (r & 7);  // global chunk for this lane's LDS slot
  }
  const int bh = wave >> 2;
  const __bf16* wcol = Wv + n0 + 128 * bh;
  auto issue = [&](int ks, int buf) {
    const int k0 = ks * kStepK;
    const uint32_t sa = lds0 + buf * kStageBytes;
#pragma unroll
    for (int p = 0; p < 4; ++p)
      dma::dma_b128_u(xrow[p] + k0 + xslot[p] * 8, sa + (32 * wave + 8 * p) * 128);
    const uint32_t sb = sa + kABytes + bh * (kBBytes / 2);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int kr = 16 * (wave & 3) + 4 * p + (lane >> 4);
      const int ch = (lane & 15) ^ swz16(kr);
      dma::dma_b128_u(wcol + (int64_t)(k0 + kr) * N + ch * 8,
                      sb + (16 * (wave & 3) + 4 * p) * 256);
    }
  };

  dma::f32x16 acc[2][4];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mb][nb][i] = 0.f;

  const int nk = Cin / kStepK;
  const int g = lane >> 4, r16 = lane & 15;
  issue(0, 0);
  for (int ks = 0; ks < nk; ++ks) {
    const int buf = ks & 1;
    // stage ks has landed (the only loads of this wave in flight) and every
    // wave is past step ks-1, whose buffer the next stage overwrites
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (ks + 1 < nk) issue(ks + 1, buf ^ 1);
    const unsigned char* As = smem + buf * kStageBytes;
    typedef __attribute__((address_space(3))) unsigned char lds_u8;
    const lds_u8* Bs = (const lds_u8*)(smem + buf * kStageBytes + kABytes + wn * (kBBytes / 2));
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      // the k order of the transposing read's B fragments: lane half hi
      // holds k = 4hi..4hi+3 and 8+4hi..8+4hi+3 of the 16-step, so the A
      // fragment takes the same two 4-element pieces of the X row
      dma::bf16x8 af[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int row = 64 * wm + 32 * mb + l32;
        const unsigned char* rp = As + row * 128 + 8 * hi;
        const dma::u32x2 a0 =
            *reinterpret_cast<const dma::u32x2*>(rp + (((2 * kk) ^ (row & 7)) << 4));
        const dma::u32x2 a1 =
            *reinterpret_cast<const dma::u32x2*>(rp + (((2 * kk + 1) ^ (row & 7)) << 4));
        const dma::u32x4 av = {a0[0], a0[1], a1[0], a1[1]};
        af[mb] = __builtin_bit_cast(dma::bf16x8, av);
      }
      const int kr = 16 * kk + 4 * (g >> 1) + (r16 >> 2);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int c0 = nb * 32 + 16 * (g & 1) + 4 * (r16 & 3);
        const int lc = c0 >> 3, byte = (c0 & 7) * 2;
        const dma::i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (dma::lds_i16x4*)(Bs + kr * 256 + ((lc ^ swz16(kr)) << 4) + byte));
        const dma::i16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (dma::lds_i16x4*)(Bs + (kr + 8) * 256 + ((lc ^ swz16(kr + 8)) << 4) + byte));
        const dma::u32x2 lo2 = __builtin_bit_cast(dma::u32x2, lo);
        const dma::u32x2 up2 = __builtin_bit_cast(dma::u32x2, up);
        const dma::u32x4 bv = {lo2[0], lo2[1], up2[0], up2[1]};
        const dma::bf16x8 bfr = __builtin_bit_cast(dma::bf16x8, bv);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mb], bfr, acc[mb][nb], 0, 0, 0);
      }
    }
  }

  // epilogue: the wave's 64 x 128 block as bf16 in LDS (rows of 256 B,
  // 16-byte chunk c of row r at c ^ (r & 15)), after every wave's last reads
  __syncthreads();
  unsigned char* Vs = smem + wave * (64 * 256);
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = 32 * mb + 8 * (i >> 2) + 4 * hi + (i & 3);
        const int col = 32 * nb + l32;
        const int ch = (col >> 3) ^ (row & 15);
        *reinterpret_cast<__bf16*>(Vs + row * 256 + (ch << 4) + (col & 7) * 2) =
            (__bf16)acc[mb][nb][i];
      }
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));  // lgkmcnt(0): own rows are in
  // stores of V: 64 rows x 256 B, one 16-byte chunk per lane, 4 rows per pass
#pragma unroll
  for (int p = 0; p < 16; ++p) {
    const int row = 4 * p + (lane >> 4), ch = lane & 15;
    const int64_t m = m0 + 64 * wm + row;
    if (m < M) {
      const int64_t b = m / Sk, j = m - b * Sk;
      const uint4 v = *reinterpret_cast<const uint4*>(Vs + row * 256 + ((ch ^ (row & 15)) << 4));
      *reinterpret_cast<uint4*>(V + b * v_sb + j * v_ss + n0 + 128 * wn + ch * 8) = v;
    }
  }
  if constexpr (EPI) {
    // partial pre over this block's 128 columns: out[r][m] = sum_n D3[r][n] V[m][n]
    // with D3 row r = split*8 + h (hi, mid, lo parts of Delta[n][h]; rows 24..31 zero)
    dma::f32x16 pacc[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) pacc[mb][i] = 0.f;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const int cg = 128 * wn + 16 * kk + 8 * hi;  // first column of this lane's 8
      const dma::bf16x8 dop =
          *reinterpret_cast<const dma::bf16x8*>(Ds + l32 * 512 + (((cg >> 3) ^ l32) << 4));
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int row = 32 * mb + l32;
        const int ch = (2 * kk + hi) ^ (row & 15);
        const dma::bf16x8 vop = *reinterpret_cast<const dma::bf16x8*>(Vs + row * 256 + (ch << 4));
        pacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dop, vop, pacc[mb], 0, 0, 0);
      }
    }
    // lane: key column m = l32 of block mb; register i = row 8(i/4) + 4hi + i%4,
    // i.e. split i/4 (3: padding), head 4hi + i%4.  The wn = 1 wave hands its
    // sums to its wn = 0 partner (same rows) through its own LDS block, whose
    // reads above are done; the partner adds them and stores.
    float4 o[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      float* op = &o[mb].x;
#pragma unroll
      for (int t = 0; t < 4; ++t) op[t] = pacc[mb][t] + (pacc[mb][4 + t] + pacc[mb][8 + t]);
    }
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));  // lgkmcnt(0)
    if (wn == 1) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        reinterpret_cast<float4*>(Vs)[(32 * mb + l32) * 2 + hi] = o[mb];
    }
    __syncthreads();
    if (wn == 0) {
      const float4* other = reinterpret_cast<const float4*>(smem + (wave + 4) * (64 * 256));
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int64_t m = m0 + 64 * wm + 32 * mb + l32;
        const float4 u = other[(32 * mb + l32) * 2 + hi];
        const float4 r = {o[mb].x + u.x, o[mb].y + u.y, o[mb].z + u.z, o[mb].w + u.w};
        if (m < M)
          *reinterpret_cast<float4*>(pre_part + ((int64_t)nt * M + m) * kHeads + 4 * hi) = r;
      }
    }
  }
}

__device__ __forceinline__ float softplus_v(float x) {
  return x > 0.f ? x + log1pf(expf(-x)) : log1pf(expf(x));
}

// delta[b,h,j] = exp(softplus(sum of the N/256 partials of pre) * A[h])
__global__ __launch_bounds__(256) void vproj_finish_kernel(const float* __restrict__ pre_part,
                                                           int64_t M, int Sk, int Hkv, int nparts,
                                                           const float* __restrict__ A,
                                                           float* __restrict__ delta) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t m = t / Hkv;
  const int h = (int)(t - m * Hkv);
  if (m >= M) return;
  float x = 0.f;
  for (int pp = 0; pp < nparts; ++pp) x += pre_part[((int64_t)pp * M + m) * kHeads + h];
  const int64_t b = m / Sk, j = m - b * Sk;
  delta[(b * Hkv + h) * Sk + j] = expf(softplus_v(x) * A[h]);
}

}  // namespace

size_t dma_vproj_ws_bytes(int64_t M, int64_t N) {
  // the partials of pre, one per column tile
  return (size_t)(N / kTileN) * (size_t)M * kHeads * 4;
}

hipError_t dma_launch_vproj(const void* X, int64_t x_sb, int64_t x_ss, const void* Wv, void* V,
                            int64_t v_sb, int64_t v_ss, int64_t B, int64_t Sk, int64_t Cin,
                            int64_t N, int64_t Hkv, const float* Delta, const float* A,
                            float* delta, void* ws, hipStream_t st) {
  const int64_t M = B * Sk;
  const int nm = (int)((M + kTileM - 1) / kTileM);
  const int nn = (int)(N / kTileN);
  const int nblocks = (nm + 7) / 8 * 8 * nn;
  const bool epi = delta != nullptr;
  float* pre = epi ? static_cast<float*>(ws) : nullptr;
  const void* fn = epi ? reinterpret_cast<const void*>(&vproj_kernel<true>)
                       : reinterpret_cast<const void*>(&vproj_kernel<false>);
  const size_t lds = epi ? (size_t)kLdsBytes : (size_t)(2 * kStageBytes);
  hipError_t e = dma_func_max_lds(fn, lds);
  if (e != hipSuccess) return e;
  if (epi)
    hipLaunchKernelGGL(vproj_kernel<true>, dim3(nblocks), dim3(kWaves * 64), lds, st,
                       static_cast<const __bf16*>(X), x_sb, x_ss, static_cast<const __bf16*>(Wv),
                       static_cast<__bf16*>(V), v_sb, v_ss, M, (int)Sk, (int)Cin, (int)N, Delta,
                       (int)Hkv, pre, nm);
  else
    hipLaunchKernelGGL(vproj_kernel<false>, dim3(nblocks), dim3(kWaves * 64), lds, st,
                       static_cast<const __bf16*>(X), x_sb, x_ss, static_cast<const __bf16*>(Wv),
                       static_cast<__bf16*>(V), v_sb, v_ss, M, (int)Sk, (int)Cin, (int)N, Delta,
                       (int)Hkv, pre, nm);
  if (epi) {
    const int64_t threads = M * Hkv;
    hipLaunchKernelGGL(vproj_finish_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                       st, pre, M, (int)Sk, (int)Hkv, (int)(N / kTileN), A, delta);
  }
  return hipGetLastError();
}
