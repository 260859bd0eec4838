// Backward of the masked attention of the DMA forward, bf16 prefill (Hugging
// Face blog "Trainable Dynamic Mask Sparse Attention", section "Efficient
// Sparse Attention Computation"; a masked key has weight exactly 0 and so
// gradient exactly 0, the section's "Backward Pass Safety" item).  Gradients
// of L = sum(dO * O) with the keep sets held fixed (they are piecewise
// constant in delta):
//   P_ij  = exp(scale q_i.k_j + delta_j - lse_i),   Dv_i = dO_i . O_i
//   dS_ij = P_ij (dO_i . v_j - Dv_i)
//   dQ_i = scale sum_j dS_ij k_j,   dK_j = scale sum_i dS_ij q_i,
//   dV_j = sum_i P_ij dO_i,         ddelta_j = sum_i dS_ij
// (i over the rows and the G query heads of the key's kv head).
//
// Kernels:
//   dq      query-major with the forward's work split: a workgroup walks the
//           compacted key list of its 64-row tile, one wave per (query head,
//           32-row half).  S^T = K Q^T and dP^T = V dO^T read K and V rows;
//           dQ^T += K^T dS^T reads K transposed.  Q^T and dO^T stay in
//           registers.  Its prologue also forms Dv_i = dO_i . O_i.  With four
//           query heads per workgroup the waves run the forward's ping-pong
//           (bwd_dq_pp_kernel), else one 64-key chunk per step.
//   dkv     key-major over groups of 512 rows (8 query tiles), in two passes
//           (dV, then dK and ddelta) so that two waves fit per SIMD.  The keys some
//           row of a group keeps (at most w + 511: the candidate lists of the
//           mask step) are cut into slices of 128, one per workgroup and 32
//           per wave, with K and V held in registers.  The workgroup streams
//           the group's 64-row tiles of Q and dO (every query head) through
//           LDS and accumulates dK^T, dV^T and ddelta, which it writes as the
//           group's partial sums.  Natural 64-key tiles would do 4x (16K
//           keys) to 8x (64K) the kept work, since the best key of a tile
//           stays kept to the end of the sequence; within a group a
//           candidate is kept on most rows.
//   reduce  key j is kept on rows [j, e_j), i.e. in groups j/512 ..
//           (e_j-1)/512; it sums its partials over those groups, finding its
//           place in each group's list through a dense (group, key) map that
//           the dkv kernel writes.
// LDS tiles are 64 rows of 256 bytes.  The 16-byte chunk c of row r is
// stored at c ^ (((r & 3) << 2) | ((r >> 2) & 3)): 16 consecutive rows put
// one chunk on 16 distinct chunk slots (row reads), and 4 consecutive rows
// put a 32-byte piece on 4 distinct 32-byte slots (transposing reads), so
// both access patterns are free of bank conflicts.
#include "lds_dma.h"

#include <algorithm>

namespace {

constexpr int kBq = 64;
constexpr int kBk = 64;
constexpr int kD = 128;
constexpr int kRowB = kD * 2;
constexpr int kTileB = 64 * kRowB;
constexpr int kGroupRows = 512;   // rows per key-side group
constexpr int kSliceKeys = 128;   // candidate keys per key-side workgroup (4 waves x 32)
constexpr float kLog2e = 1.4426950408889634f;

using dma::dma_b128;
using dma::dma_b32;
using dma::i16x4;
using dma::lds_addr;
using dma::lds_i16x4;
using dma::to_bf16x8;
using dma::u32x2;
using dma::u32x4;
typedef __attribute__((address_space(3))) unsigned char lds_u8;

__device__ __forceinline__ int swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

// All of this wave's direct loads have landed; then the workgroup barrier.
__device__ __forceinline__ void wait_all_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0);  // vmcnt(0) expcnt(0) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// A or B operand of a 32x32x16 MFMA read along a tile row: row `row`,
// logical 16-byte chunk lc (elements 8*lc .. 8*lc+7).
__device__ __forceinline__ dma::bf16x8 row_operand(const unsigned char* tile, int row, int lc) {
  return *reinterpret_cast<const dma::bf16x8*>(tile + row * kRowB + ((lc ^ swz(row)) << 4));
}

// A operand of an MFMA that contracts over 16 tile rows: element (m, k) =
// tile[row(k)][dbase + m] for m = lane % 32 and k = 8*hi + t, where row(k) is
// rbase + 4*hi + t for t < 4 and rbase + 8 + 4*hi + (t - 4) otherwise: the
// row order of the B operands built from a 32x32 accumulator (register i of
// lane (l32, hi) holds row 8*(i/4) + 4*hi + i%4).  Two transposing reads: a
// 16-lane group g addresses rows rbase + 4*(g/2) + r/4 (and 8 rows further),
// columns dbase + 16*(g%2) + 4*(r%4), and lane i of the group receives the
// 4 rows of column dbase + 16*(g%2) + i.
__device__ __forceinline__ dma::bf16x8 tr_operand(const unsigned char* tile, int rbase, int dbase,
                                                  int lane) {
  const int g = lane >> 4, r = lane & 15;
  const int k0 = rbase + 4 * (g >> 1) + (r >> 2);
  const int d0 = dbase + 16 * (g & 1) + 4 * (r & 3);
  const int lc = d0 >> 3, byte = (d0 & 7) * 2;
  const lds_u8* base = (const lds_u8*)tile;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(base + k0 * kRowB + ((lc ^ swz(k0)) << 4) + byte));
  const i16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(base + (k0 + 8) * kRowB + ((lc ^ swz(k0 + 8)) << 4) + byte));
  const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), up2 = __builtin_bit_cast(u32x2, up);
  const u32x4 vv = {lo2[0], lo2[1], up2[0], up2[1]};
  return __builtin_bit_cast(dma::bf16x8, vv);
}

__device__ __forceinline__ dma::f32x16 mfma(dma::bf16x8 a, dma::bf16x8 b, dma::f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- dq
struct DqSmem {
  unsigned char k[2][kTileB];  // K chunk tiles (gathered rows)
  unsigned char v[2][kTileB];  // V chunk tiles
  int jl[3][kBk];              // list entries: chunk c in slot c % 3
  float dl[2][kBk];            // delta of chunk c's keys in slot c % 2
  int ev[2][kBk];              // their eviction rows
};

template <int NH>
__global__ __launch_bounds__(NH * 128, 2) void bwd_dq_kernel(DmaBwdArgs a) {
  constexpr int NW = NH * 2;
  __shared__ __align__(16) DqSmem sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const DmaAttnArgs& f = a.f;
  const int G = (int)(f.Hq / f.Hkv);
  const int ngrp = G / NH;
  const int t = blockIdx.x, h = blockIdx.y;
  const int b = blockIdx.z / ngrp, hgrp = blockIdx.z % ngrp;
  const int hq = h * G + hgrp * NH + (wave >> 1);
  const int half = wave & 1;
  const int64_t seg = (int64_t)b * f.Hkv + h;
  const int64_t g = seg * f.n_tiles + t;
  const int r_lo = t * kBq;
  const int rows = min(kBq, (int)f.Sq - r_lo);
  const int cnt = f.u_cnt[g];
  const int32_t* list = f.u_idx + g * f.u_stride;
  const float* dlg = f.delta + seg * f.Sk;
  const int32_t* evg = f.evict + seg * f.Sk;
  const int nch = (cnt + kBk - 1) / kBk;
  const int clast = max(cnt - 1, 0);
  const unsigned char* Kg = static_cast<const unsigned char*>(f.K) + (b * f.ksb + h * f.ksh) * 2;
  const unsigned char* Vg = static_cast<const unsigned char*>(f.V) + (b * f.ksb + h * f.ksh) * 2;
  const uint32_t rowb = (uint32_t)(f.kss * 2);
  const float scale2 = f.scale * kLog2e;

  // this lane's query column n, its Q^T and dO^T operands, lse and Dv
  const int n = half * 32 + l32;
  const int nr = r_lo + (n < rows ? n : 0);  // rows past the tile repeat its first row
  const int pos = (int)f.q0 + r_lo + n;
  dma::bf16x8 qf[8], gf[8];
  {
    const uint16_t* qrow =
        static_cast<const uint16_t*>(f.Q) + b * f.qsb + hq * f.qsh + (int64_t)nr * f.qss;
    const uint16_t* grow = static_cast<const uint16_t*>(a.dO) + ((b * f.Sq + nr) * f.Hq + hq) * kD;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      qf[kk] = __builtin_bit_cast(dma::bf16x8,
                                  *reinterpret_cast<const u32x4*>(qrow + kk * 16 + hi * 8));
      gf[kk] = __builtin_bit_cast(dma::bf16x8,
                                  *reinterpret_cast<const u32x4*>(grow + kk * 16 + hi * 8));
    }
  }
  // the row's weights are exp(scale q.k + delta - lse): delta - lse is taken
  // first, exact for every key near the row's maximum whatever the range of
  // delta, so the logits carried stay small
  const float lse_q = f.lse[((int64_t)b * f.Hq + hq) * f.Sq + nr];
  // D_i = dO_i . O_i: this lane's 64 of the row's 128 values against the dO^T
  // operand it holds, then the other half from lane ^ 32.  O + O_res (when
  // given) restores the forward's fp32 O.  Every (row, query head) belongs to
  // exactly one wave, which stores D_i for the key-major passes.
  float dv_q;
  {
    const int64_t ro = ((b * f.Sq + nr) * f.Hq + hq) * kD + hi * 8;
    const uint16_t* orow = static_cast<const uint16_t*>(f.O) + ro;
    const uint16_t* rrow = static_cast<const uint16_t*>(f.ores) + ro;
    u32x4 ov[8], rv[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      ov[kk] = *reinterpret_cast<const u32x4*>(orow + kk * 16);
      rv[kk] = f.ores ? *reinterpret_cast<const u32x4*>(rrow + kk * 16) : u32x4{0u, 0u, 0u, 0u};
    }
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const u32x4 gv = __builtin_bit_cast(u32x4, gf[kk]);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc[e] += (dma::bf16_lo(ov[kk][e]) + dma::bf16_lo(rv[kk][e])) * dma::bf16_lo(gv[e]) +
                  (dma::bf16_hi(ov[kk][e]) + dma::bf16_hi(rv[kk][e])) * dma::bf16_hi(gv[e]);
    }
    const float part = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    dv_q = part + __shfl_xor(part, 32);
    if (hi == 0 && n < rows) a.Dv[((int64_t)b * f.Hq + hq) * f.Sq + r_lo + n] = dv_q;
  }

  const uint32_t lds_k = lds_addr(&sm.k[0][0]), lds_v = lds_addr(&sm.v[0][0]);
  const uint32_t lds_j = lds_addr(&sm.jl[0][0]), lds_d = lds_addr(&sm.dl[0][0]),
                 lds_e = lds_addr(&sm.ev[0][0]);
  // the K and V rows of chunk x into buffer x % 2: 16 pieces of 4 rows per
  // tile, piece p by wave p % NW; lane L fills row 4p + L/16, chunk slot L%16
  auto gather = [&](int x) {
    const int buf = x & 1;
    // recomputed on every call: hoisted out of the loop, these lane constants
    // would be held (and spilled) across it
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int u = 0; u < 16 / NW; ++u) {
      const int piece = wave + u * NW;
      const int row = piece * 4 + (ln >> 4);
      const int lc = (ln & 15) ^ swz(row);
      const uint32_t j = (uint32_t)sm.jl[x % 3][row];
      dma_b128(Kg + j * rowb + lc * 16, lds_k + buf * kTileB + piece * 1024);
      dma_b128(Vg + j * rowb + lc * 16, lds_v + buf * kTileB + piece * 1024);
    }
    if (wave == 0) {
      const int j = sm.jl[x % 3][lane];
      dma_b32(dlg + j, lds_d + buf * 256);
      dma_b32(evg + j, lds_e + buf * 256);
    }
  };

  // prologue: list entries of chunks 0 and 1, then chunk 0's rows
  if (wave == 0) {
    dma_b32(list + min(lane, clast), lds_j);
    dma_b32(list + min(kBk + lane, clast), lds_j + 256);
  }
  wait_all_barrier();
  gather(0);
  wait_all_barrier();

  dma::f32x16 dq[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dq[db][i] = 0.f;

  for (int c = 0; c < nch; ++c) {
    // chunk c+2's list entries and chunk c+1's rows go out first
    if (wave == 0) dma_b32(list + min((c + 2) * kBk + lane, clast), lds_j + ((c + 2) % 3) * 256);
    if (c + 1 < nch) gather(c + 1);

    const unsigned char* KT = sm.k[c & 1];
    const unsigned char* VT = sm.v[c & 1];
    // one 32-key block at a time: S^T = K Q^T and dP^T = V dO^T (two
    // interleaved accumulator chains; lane (l32, hi) reads key row mb*32 + l32),
    // then dS^T = P^T (dP^T - Dv) as bf16 B operands; register i of the block
    // is key mb*32 + 8(i/4) + 4hi + i%4
    dma::bf16x8 dsb[2][2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      dma::f32x16 s, dp;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s[i] = 0.f;
        dp[i] = 0.f;
      }
      const int row = mb * 32 + l32;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        s = mfma(row_operand(KT, row, 2 * kk + hi), qf[kk], s);
        dp = mfma(row_operand(VT, row, 2 * kk + hi), gf[kk], dp);
      }
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        float ds[8];
#pragma unroll
        for (int h4 = 0; h4 < 2; ++h4) {
          // registers 4*q4 .. 4*q4+3 are keys kb .. kb+3
          const int q4 = 2 * hf + h4;
          const int kb = mb * 32 + 8 * q4 + 4 * hi;
          const int4 j4 = *reinterpret_cast<const int4*>(&sm.jl[c % 3][kb]);
          const int4 e4 = *reinterpret_cast<const int4*>(&sm.ev[c & 1][kb]);
          const float4 d4 = *reinterpret_cast<const float4*>(&sm.dl[c & 1][kb]);
          const int jv[4] = {j4.x, j4.y, j4.z, j4.w};
          const int ev[4] = {e4.x, e4.y, e4.z, e4.w};
          const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = 4 * q4 + r;
            // list padding (positions past cnt) and rows outside [j, e) get weight 0
            const bool kept = (c * kBk + kb + r < cnt) &
                              ((uint32_t)(pos - jv[r]) < (uint32_t)(ev[r] - jv[r]));
            const float v = fmaf(s[i], scale2, (dv[r] - lse_q) * kLog2e);
            const float p = __builtin_amdgcn_exp2f(kept ? v : -INFINITY);
            ds[4 * h4 + r] = p * (dp[i] - dv_q);
          }
        }
        dsb[mb][hf] = to_bf16x8(ds);
      }
    }
    // dQ^T += K^T dS^T: k-step (mb, hf) covers keys mb*32 + 16*hf + [0, 16)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int db = 0; db < 4; ++db)
          dq[db] = mfma(tr_operand(KT, mb * 32 + 16 * hf, db * 32, lane), dsb[mb][hf], dq[db]);
    wait_all_barrier();
  }
  __builtin_amdgcn_s_waitcnt(0);

  if (n < rows) {
    float* orow = a.dQ + (((int64_t)b * f.Sq + r_lo + n) * f.Hq + hq) * kD;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = db * 32 + 8 * q4 + 4 * hi;
        float4 o;
        o.x = f.scale * dq[db][4 * q4 + 0];
        o.y = f.scale * dq[db][4 * q4 + 1];
        o.z = f.scale * dq[db][4 * q4 + 2];
        o.w = f.scale * dq[db][4 * q4 + 3];
        *reinterpret_cast<float4*>(orow + d) = o;
      }
  }
}

// ---------------------------------------------------------------- dq, ping-pong
// The same gradient, for four query heads per workgroup (8 waves, one of each
// group per SIMD), with the forward's ping-pong.  A step is one 32-key block
// b (chunk b/2, half b%2).  Per block a wave runs an MFMA phase
//   M_b = { dQ^T += K^T dS^T of block b-1 ;  S^T, dP^T of block b }
// and a VALU phase
//   V_b = { dS^T of block b from S^T and dP^T }.
// In step b group A (waves 0-3) runs M_b then V_b; group B (waves 4-7) runs
// V_{b-1} then M_b, so one wave of every SIMD mostly multiplies while the
// other mostly exponentiates.  One workgroup barrier ends each step.
//
// Memory: K of chunk c sits in buffer c % 3 (read by the S products of its
// two blocks and by their dQ products one step later), V of chunk c in
// c % 2, list entries in slot c % 4, delta and eviction rows in c % 3.  At
// the start of step 2c the waves gather chunk c+1 (K, V rows, delta and
// eviction rows) and wave 0 loads the list entries of chunk c+2; the barrier
// ending step 2c+1 waits for them (two steps in flight), and every buffer a
// step writes was last read two steps or more before it.
struct DqPpSmem {
  unsigned char k[3][kTileB];  // K of chunk c in buffer c % 3
  unsigned char v[2][kTileB];  // V of chunk c in buffer c % 2
  int jl[4][kBk];              // list entries of chunk c in slot c % 4
  float dl[3][kBk];            // delta of chunk c's keys in slot c % 3
  int ev[3][kBk];              // their eviction rows
};

// End of a ping-pong step: the LDS reads of this wave are done, and at the
// steps that close a load window (LOADS) its direct loads have landed too.
template <bool LOADS>
__device__ __forceinline__ void pp_barrier() {
  asm volatile("" ::: "memory");
#ifdef DMA_SAFE_SYNC
  __builtin_amdgcn_s_waitcnt(0);  // vmcnt(0) expcnt(0) lgkmcnt(0)
#else
  if constexpr (LOADS)
    __builtin_amdgcn_s_waitcnt(0);  // vmcnt(0) expcnt(0) lgkmcnt(0)
  else
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));  // lgkmcnt(0) only
#endif
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__global__ __launch_bounds__(512, 2) void bwd_dq_pp_kernel(DmaBwdArgs a) {
  constexpr int NH = 4, NW = 8;
  __shared__ __align__(16) DqPpSmem sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const DmaAttnArgs& f = a.f;
  const int G = (int)(f.Hq / f.Hkv);
  const int ngrp = G / NH;
  const int t = blockIdx.x, h = blockIdx.y;
  const int b = blockIdx.z / ngrp, hgrp = blockIdx.z % ngrp;
  const int hq = h * G + hgrp * NH + (wave >> 1);
  const int half = wave & 1;
  const bool grp_a = wave < NW / 2;
  const int64_t seg = (int64_t)b * f.Hkv + h;
  const int64_t g = seg * f.n_tiles + t;
  const int r_lo = t * kBq;
  const int rows = min(kBq, (int)f.Sq - r_lo);
  const int cnt = f.u_cnt[g];
  const int32_t* list = f.u_idx + g * f.u_stride;
  const float* dlg = f.delta + seg * f.Sk;
  const int32_t* evg = f.evict + seg * f.Sk;
  const int nch = (cnt + kBk - 1) / kBk;
  const int nb = 2 * nch;  // 32-key blocks
  const int clast = max(cnt - 1, 0);
  const unsigned char* Kg = static_cast<const unsigned char*>(f.K) + (b * f.ksb + h * f.ksh) * 2;
  const unsigned char* Vg = static_cast<const unsigned char*>(f.V) + (b * f.ksb + h * f.ksh) * 2;
  const uint32_t rowb = (uint32_t)(f.kss * 2);
  const float scale2 = f.scale * kLog2e;

  // this lane's query column n, its Q^T and dO^T operands, lse and D_i
  const int n = half * 32 + l32;
  const int nr = r_lo + (n < rows ? n : 0);  // rows past the tile repeat its first row
  const int pos = (int)f.q0 + r_lo + n;
  dma::bf16x8 qf[8], gf[8];
  {
    const uint16_t* qrow =
        static_cast<const uint16_t*>(f.Q) + b * f.qsb + hq * f.qsh + (int64_t)nr * f.qss;
    const uint16_t* grow = static_cast<const uint16_t*>(a.dO) + ((b * f.Sq + nr) * f.Hq + hq) * kD;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      qf[kk] = __builtin_bit_cast(dma::bf16x8,
                                  *reinterpret_cast<const u32x4*>(qrow + kk * 16 + hi * 8));
      gf[kk] = __builtin_bit_cast(dma::bf16x8,
                                  *reinterpret_cast<const u32x4*>(grow + kk * 16 + hi * 8));
    }
  }
  const float lse_q = f.lse[((int64_t)b * f.Hq + hq) * f.Sq + nr];
  // D_i = dO_i . O_i, as in bwd_dq_kernel
  float dv_q;
  {
    const int64_t ro = ((b * f.Sq + nr) * f.Hq + hq) * kD + hi * 8;
    const uint16_t* orow = static_cast<const uint16_t*>(f.O) + ro;
    const uint16_t* rrow = static_cast<const uint16_t*>(f.ores) + ro;
    u32x4 ov[8], rv[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      ov[kk] = *reinterpret_cast<const u32x4*>(orow + kk * 16);
      rv[kk] = f.ores ? *reinterpret_cast<const u32x4*>(rrow + kk * 16) : u32x4{0u, 0u, 0u, 0u};
    }
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const u32x4 gv = __builtin_bit_cast(u32x4, gf[kk]);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc[e] += (dma::bf16_lo(ov[kk][e]) + dma::bf16_lo(rv[kk][e])) * dma::bf16_lo(gv[e]) +
                  (dma::bf16_hi(ov[kk][e]) + dma::bf16_hi(rv[kk][e])) * dma::bf16_hi(gv[e]);
    }
    const float part = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    dv_q = part + __shfl_xor(part, 32);
    if (hi == 0 && n < rows) a.Dv[((int64_t)b * f.Hq + hq) * f.Sq + r_lo + n] = dv_q;
  }

  const uint32_t lds_k = lds_addr(&sm.k[0][0]), lds_v = lds_addr(&sm.v[0][0]);
  const uint32_t lds_j = lds_addr(&sm.jl[0][0]), lds_d = lds_addr(&sm.dl[0][0]),
                 lds_e = lds_addr(&sm.ev[0][0]);
  // chunk x's K and V rows (16 pieces of 4 rows per tile, piece p by wave
  // p % NW; lane L fills row 4p + L/16, chunk slot L%16), and wave 0 its
  // delta and eviction rows
  auto gather = [&](int x) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int kb = x % 3, vb = x & 1, js = x & 3, ds_ = x % 3;
#pragma unroll
    for (int u = 0; u < 16 / NW; ++u) {
      const int piece = wave + u * NW;
      const int row = piece * 4 + (ln >> 4);
      const int lc = (ln & 15) ^ swz(row);
      const uint32_t j = (uint32_t)sm.jl[js][row];
      dma_b128(Kg + j * rowb + lc * 16, lds_k + kb * kTileB + piece * 1024);
      dma_b128(Vg + j * rowb + lc * 16, lds_v + vb * kTileB + piece * 1024);
    }
    if (wave == 0) {
      const int j = sm.jl[js][lane];
      dma_b32(dlg + j, lds_d + ds_ * 256);
      dma_b32(evg + j, lds_e + ds_ * 256);
    }
  };
  // the loads of step b (even steps only): list entries of chunk b/2 + 2, chunk b/2 + 1
  auto issue = [&](int bb) {
    if ((bb & 1) == 0) {
      const int c = bb >> 1;
      if (c < nch) {
        if (wave == 0) dma_b32(list + min((c + 2) * kBk + lane, clast), lds_j + ((c + 2) & 3) * 256);
        if (c + 1 < nch) gather(c + 1);
      }
    }
  };

  // prologue: list entries of chunks 0 and 1, then chunk 0's rows
  if (wave == 0) {
    dma_b32(list + min(lane, clast), lds_j);
    dma_b32(list + min(kBk + lane, clast), lds_j + 256);
  }
  wait_all_barrier();
  gather(0);
  wait_all_barrier();

  dma::f32x16 dq[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dq[db][i] = 0.f;
  dma::f32x16 s, dp;
  dma::bf16x8 dsb[2];

  // M_bb: dQ of block bb-1 (from dsb), then S^T and dP^T of block bb (lane
  // (l32, hi) reads key row mb*32 + l32; register i is key mb*32 + 8(i/4) +
  // 4hi + i%4)
  auto mphase = [&](int bb) {
    if (bb >= 1) {
      const int pbk = bb - 1;
      const unsigned char* KP = sm.k[(pbk >> 1) % 3];
      const int pmb = pbk & 1;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int db = 0; db < 4; ++db)
          dq[db] = mfma(tr_operand(KP, pmb * 32 + 16 * hf, db * 32, lane), dsb[hf], dq[db]);
    }
    if (bb < nb) {
      const int cb = bb >> 1, mb = bb & 1;
      const unsigned char* KT = sm.k[cb % 3];
      const unsigned char* VT = sm.v[cb & 1];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s[i] = 0.f;
        dp[i] = 0.f;
      }
      const int row = mb * 32 + l32;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        s = mfma(row_operand(KT, row, 2 * kk + hi), qf[kk], s);
        dp = mfma(row_operand(VT, row, 2 * kk + hi), gf[kk], dp);
      }
    }
  };
  // V_bb: dS^T = P^T (dP^T - D) of block bb as bf16 B operands.  The
  // exponent is scale2 * s + log2(e) * delta - log2(e) * lse: two FMAs per
  // element.  MASKED blocks test j <= p < e_j and the list's end per element;
  // the others (the leading chunks, whose keys every row of the tile keeps)
  // need no test.
  const float nl = -lse_q * kLog2e;
  auto vphase = [&](int bb, auto masked) {
    constexpr bool MASKED = decltype(masked)::value;
    const int cb = bb >> 1, mb = bb & 1;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      float ds[8];
#pragma unroll
      for (int h4 = 0; h4 < 2; ++h4) {
        const int q4 = 2 * hf + h4;
        const int kb = mb * 32 + 8 * q4 + 4 * hi;
        const float4 d4 = *reinterpret_cast<const float4*>(&sm.dl[cb % 3][kb]);
        const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
        int jv[4] = {0, 0, 0, 0}, ev[4] = {0, 0, 0, 0};
        if constexpr (MASKED) {
          const int4 j4 = *reinterpret_cast<const int4*>(&sm.jl[cb & 3][kb]);
          const int4 e4 = *reinterpret_cast<const int4*>(&sm.ev[cb % 3][kb]);
          jv[0] = j4.x; jv[1] = j4.y; jv[2] = j4.z; jv[3] = j4.w;
          ev[0] = e4.x; ev[1] = e4.y; ev[2] = e4.z; ev[3] = e4.w;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 4 * q4 + r;
          float v = fmaf(s[i], scale2, fmaf(dv[r], kLog2e, nl));
          if constexpr (MASKED) {
            // list padding (positions past cnt) and rows outside [j, e) get weight 0
            const bool kept = (cb * kBk + kb + r < cnt) &
                              ((uint32_t)(pos - jv[r]) < (uint32_t)(ev[r] - jv[r]));
            v = kept ? v : -INFINITY;
          }
          const float p = __builtin_amdgcn_exp2f(v);
          ds[4 * h4 + r] = p * (dp[i] - dv_q);
        }
      }
      dsb[hf] = to_bf16x8(ds);
    }
  };
  using Plain = std::integral_constant<bool, false>;
  using Masked = std::integral_constant<bool, true>;
  // blocks [0, pb) belong to chunks every row keeps
  const int pb = 2 * min(f.u_nfull[g] / kBk, nch);

  if (grp_a) {
    int bb = 0;
    for (; bb < pb; ++bb) {
      issue(bb);
      mphase(bb);
      vphase(bb, Plain{});
      if (bb & 1)
        pp_barrier<true>();
      else
        pp_barrier<false>();
    }
    for (; bb <= nb; ++bb) {
      issue(bb);
      mphase(bb);
      if (bb < nb) vphase(bb, Masked{});
      if (bb & 1)
        pp_barrier<true>();
      else
        pp_barrier<false>();
    }
  } else {
    int bb = 0;
    for (; bb <= pb; ++bb) {
      issue(bb);
      if (bb >= 1) vphase(bb - 1, Plain{});
      mphase(bb);
      if (bb & 1)
        pp_barrier<true>();
      else
        pp_barrier<false>();
    }
    for (; bb <= nb; ++bb) {
      issue(bb);
      vphase(bb - 1, Masked{});
      mphase(bb);
      if (bb & 1)
        pp_barrier<true>();
      else
        pp_barrier<false>();
    }
  }
  __builtin_amdgcn_s_waitcnt(0);

  // dQ goes out through LDS (the K/V buffers, free after the last barrier)
  // in two halves of 64 columns, so that each store instruction writes whole
  // 256-byte row pieces (16 bytes per lane, 16 lanes per row) instead of 16
  // bytes in each of 32 rows
  __syncthreads();
  constexpr int kOutRowB = 256 + 16;
  static_assert(8 * 32 * kOutRowB <= (int)(sizeof(sm.k) + sizeof(sm.v)), "dQ staging fits");
  unsigned char* ow = &sm.k[0][0] + wave * (32 * kOutRowB);
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
    for (int db = 2 * h2; db < 2 * h2 + 2; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int dl = (db - 2 * h2) * 32 + 8 * q4 + 4 * hi;
        float4 o;
        o.x = f.scale * dq[db][4 * q4 + 0];
        o.y = f.scale * dq[db][4 * q4 + 1];
        o.z = f.scale * dq[db][4 * q4 + 2];
        o.w = f.scale * dq[db][4 * q4 + 3];
        *reinterpret_cast<float4*>(ow + l32 * kOutRowB + dl * 4) = o;
      }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int r = it * 4 + (lane >> 4);  // the wave's row r: query half*32 + r
      const float4 v = *reinterpret_cast<const float4*>(ow + r * kOutRowB + (lane & 15) * 16);
      if (half * 32 + r < rows)
        *reinterpret_cast<float4*>(a.dQ + (((int64_t)b * f.Sq + r_lo + half * 32 + r) * f.Hq + hq) * kD +
                                   h2 * 64 + (lane & 15) * 4) = v;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

// ---------------------------------------------------------------- dkv
struct DkvSmem {
  unsigned char q[2][kTileB];   // Q rows of one (row tile, query head)
  unsigned char g[2][kTileB];   // dO rows
  float lse[2][64];
  float dv[2][64];
  int alive[4];
};

// MODE 0 accumulates dV (from P), MODE 1 dK and ddelta (from dS).  Split in
// two passes, each wave holds one accumulator block (64 registers) and at most
// two stationary operand sets, so two waves fit per SIMD; together the passes
// redo the score product once more.
template <int MODE>
__global__ __launch_bounds__(256, 2) void bwd_dkv_kernel(DmaBwdArgs a) {
  __shared__ __align__(16) DkvSmem sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const DmaAttnArgs& f = a.f;
  const int G = (int)(f.Hq / f.Hkv);
  const int slice = blockIdx.x, grp = blockIdx.y;
  const int64_t seg = blockIdx.z;
  const int b = (int)(seg / f.Hkv), h = (int)(seg % f.Hkv);
  const int64_t gi = seg * a.n_super + grp;
  const int count = a.ccnt[gi];
  if (slice * kSliceKeys >= count) return;
  const int32_t* cj = a.cj + gi * a.cap;
  const int32_t* ce = a.ce + gi * a.cap;
  const int slot = slice * kSliceKeys + wave * 32 + l32;
  const bool real = slot < count;
  const int sl = min(slot, count - 1);
  const int j = cj[sl];
  const int p_end = (int)(f.q0 + f.Sq);
  // padding lanes get an empty row range, so they never count
  const int e = real ? min(ce[sl], p_end) : j;
  const float dlt = f.delta[seg * f.Sk + j];
  // K^T (and, for dK, V^T) operands of this lane's key: K[j][kk*16 + 8*hi + 0..7]
  dma::bf16x8 kf[8], vf[8];
  {
    const uint16_t* krow = static_cast<const uint16_t*>(f.K) + b * f.ksb + h * f.ksh + (int64_t)j * f.kss;
    const uint16_t* vrow = static_cast<const uint16_t*>(f.V) + b * f.ksb + h * f.ksh + (int64_t)j * f.kss;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      kf[kk] = __builtin_bit_cast(dma::bf16x8,
                                  *reinterpret_cast<const u32x4*>(krow + kk * 16 + hi * 8));
      if constexpr (MODE == 1)
        vf[kk] = __builtin_bit_cast(dma::bf16x8,
                                    *reinterpret_cast<const u32x4*>(vrow + kk * 16 + hi * 8));
    }
  }
  // row tiles of the group in which some key of the slice is kept
  const int g_lo = grp * kGroupRows;                          // first row (relative to q0)
  const int ntile = min(kGroupRows, (int)f.Sq - g_lo + kBq - 1) / kBq;
  int am = 0;
  for (int rt = 0; rt < ntile; ++rt) {
    const int p_lo = (int)f.q0 + g_lo + rt * kBq;
    const int p_hi = min(p_lo + kBq, p_end) - 1;
    if (j <= p_hi && e > max(j, p_lo)) am |= 1 << rt;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) am |= __shfl_xor(am, o);
  if (lane == 0) sm.alive[wave] = am;
  __syncthreads();
  const int alive = sm.alive[0] | sm.alive[1] | sm.alive[2] | sm.alive[3];
  const int nt = __popc(alive);
  const int nsteps = nt * G;

  const float scale2 = f.scale * kLog2e;
  const float dltl = dlt * kLog2e;
  const uint32_t span = (uint32_t)(e - j);
  const uint32_t lds_q = lds_addr(&sm.q[0][0]), lds_g = lds_addr(&sm.g[0][0]);
  const uint32_t lds_l = lds_addr(&sm.lse[0][0]), lds_dv = lds_addr(&sm.dv[0][0]);
  // step st = (k-th alive row tile, head st % G)
  auto tile_of = [&](int st) {
    int k = st / G, m = alive;
    for (int u = 0; u < k; ++u) m &= m - 1;
    return __builtin_ctz(m);
  };
  // Q and dO rows of step st into buffer st % 2: 16 pieces of 4 rows per tile,
  // piece p by wave p % 4; rows past the sequence repeat its last row
  auto stage = [&](int st) {
    const int buf = st & 1;
    const int rt = tile_of(st);
    const int hq = h * G + st % G;
    const int r0 = g_lo + rt * kBq;
    const unsigned char* Qb = static_cast<const unsigned char*>(f.Q) + (b * f.qsb + hq * f.qsh) * 2;
    const unsigned char* Gb = static_cast<const unsigned char*>(a.dO) + ((int64_t)b * f.Sq * f.Hq + hq) * kD * 2;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int piece = wave + u * 4;
      const int row = piece * 4 + (lane >> 4);
      const int lc = (lane & 15) ^ swz(row);
      const uint32_t r = (uint32_t)min(r0 + row, (int)f.Sq - 1);
      dma_b128(Qb + r * (uint32_t)(f.qss * 2) + lc * 16, lds_q + buf * kTileB + piece * 1024);
      dma_b128(Gb + r * (uint32_t)(f.Hq * kD * 2) + lc * 16, lds_g + buf * kTileB + piece * 1024);
    }
    if (wave < 2) {
      const int r = min(r0 + lane, (int)f.Sq - 1);
      const int64_t o = ((int64_t)b * f.Hq + hq) * f.Sq + r;
      if (wave == 0)
        dma_b32(f.lse + o, lds_l + buf * 256);
      else
        dma_b32(a.Dv + o, lds_dv + buf * 256);
    }
  };

  dma::f32x16 acc[4];  // dV^T (MODE 0) or dK^T (MODE 1)
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;
  float dd = 0.f;

  if (nsteps > 0) stage(0);
  wait_all_barrier();
  for (int st = 0; st < nsteps; ++st) {
    if (st + 1 < nsteps) stage(st + 1);
    const int buf = st & 1;
    const int rt = tile_of(st);
    const int p0 = (int)f.q0 + g_lo + rt * kBq;
    const int pj0 = p0 - j;  // this lane's key against the tile's first row
    const unsigned char* QT = sm.q[buf];
    const unsigned char* GT = sm.g[buf];
#pragma unroll
    for (int rh = 0; rh < 2; ++rh) {
      dma::f32x16 s, dp;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s[i] = 0.f;
        dp[i] = 0.f;
      }
      // S = Q K^T (and dP = dO V^T) (rows x keys): lane (l32, hi) reads row rh*32 + l32
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const int row = rh * 32 + l32;
        s = mfma(row_operand(QT, row, 2 * kk + hi), kf[kk], s);
        if constexpr (MODE == 1) dp = mfma(row_operand(GT, row, 2 * kk + hi), vf[kk], dp);
      }
      // register i: row rh*32 + 8(i/4) + 4hi + i%4 of this lane's key
      dma::bf16x8 ob[2];  // P (MODE 0) or dS (MODE 1) as B operands
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float pv[8], dsv[8];
#pragma unroll
        for (int q4 = 0; q4 < 2; ++q4) {
          const int rb = rh * 32 + 16 * kb + 8 * q4 + 4 * hi;
          const float4 lv = *reinterpret_cast<const float4*>(&sm.lse[buf][rb]);
          const float4 dvv = *reinterpret_cast<const float4*>(&sm.dv[buf][rb]);
          const float lr[4] = {lv.x, lv.y, lv.z, lv.w};
          const float dr[4] = {dvv.x, dvv.y, dvv.z, dvv.w};
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int i = kb * 8 + q4 * 4 + r4;
            // kept iff j <= p < e: one unsigned compare of p - j against e - j
            const bool kept = (uint32_t)(pj0 + rb + r4) < span;
            // exponent scale2 * s + log2(e) * (delta - lse): two FMAs
            const float v = fmaf(s[i], scale2, fmaf(lr[r4], -kLog2e, dltl));
            const float pp = __builtin_amdgcn_exp2f(kept ? v : -INFINITY);
            if constexpr (MODE == 0) {
              pv[q4 * 4 + r4] = pp;
            } else {
              const float ds = pp * (dp[i] - dr[r4]);
              dsv[q4 * 4 + r4] = ds;
              dd += ds;
            }
          }
        }
        ob[kb] = to_bf16x8(MODE == 0 ? pv : dsv);
      }
      // dV^T += dO^T P, or dK^T += Q^T dS, over this half's two 16-row k-steps
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int db = 0; db < 4; ++db)
          acc[db] = mfma(tr_operand(MODE == 0 ? GT : QT, rh * 32 + 16 * kb, db * 32, lane),
                         ob[kb], acc[db]);
    }
    wait_all_barrier();
  }

  // partial sums of this group for the lane's key; register i of block db is
  // d = db*32 + 8(i/4) + 4hi + i%4
  dd += __shfl_xor(dd, 32);
  // The wave's 32 partial rows are consecutive slots, i.e. 16 KB of
  // contiguous memory: they go out through LDS (the Q/dO buffers, free after
  // the last barrier) in two halves of 64 columns, 16 bytes per lane and 16
  // lanes per 256-byte row piece, instead of 16 bytes in each of 32 rows
  {
    constexpr int kOutRowB = 256 + 16;
    static_assert(4 * 32 * kOutRowB <= (int)(sizeof(sm.q) + sizeof(sm.g)), "partial staging fits");
    unsigned char* ow = &sm.q[0][0] + wave * (32 * kOutRowB);
    float* outw = (MODE == 0 ? a.pv : a.pk) + (gi * a.cap + slice * kSliceKeys + wave * 32) * kD;
    const float sc = MODE == 0 ? 1.f : f.scale;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
      for (int db = 2 * h2; db < 2 * h2 + 2; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int dl = (db - 2 * h2) * 32 + 8 * q4 + 4 * hi;
          float4 x;
          x.x = sc * acc[db][4 * q4 + 0];
          x.y = sc * acc[db][4 * q4 + 1];
          x.z = sc * acc[db][4 * q4 + 2];
          x.w = sc * acc[db][4 * q4 + 3];
          *reinterpret_cast<float4*>(ow + l32 * kOutRowB + dl * 4) = x;
        }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int r = it * 4 + (lane >> 4);  // the wave's key r: slot slice*128 + wave*32 + r
        const float4 v = *reinterpret_cast<const float4*>(ow + r * kOutRowB + (lane & 15) * 16);
        if (slice * kSliceKeys + wave * 32 + r < count)
          *reinterpret_cast<float4*>(outw + r * kD + h2 * 64 + (lane & 15) * 4) = v;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }
  if (real) {
    const int64_t o = gi * a.cap + slot;
    if (MODE == 1 && hi == 0) {
      a.pd[o] = dd;
      a.pmap[gi * f.Sk + j] = slot;
    }
  }
}

// ---------------------------------------------------------------- reduce
// One wave per key: lane L sums d = 2L, 2L+1 over the key's groups; the
// groups' partial rows are independent loads, up to kRedBatch groups in
// flight (a key is kept on ~w rows, so most keys take one batch).
constexpr int kRedBatch = 8;
__global__ __launch_bounds__(256) void bwd_reduce_kernel(DmaBwdArgs a) {
  const DmaAttnArgs& f = a.f;
  const int64_t seg = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (j >= f.Sk) return;
  const int b = (int)(seg / f.Hkv), h = (int)(seg % f.Hkv);
  const int e = f.evict[seg * f.Sk + j];
  // rows (relative to q0) on which key j is kept
  const int r0 = max(j, (int)f.q0) - (int)f.q0;
  const int r1 = min(e, (int)(f.q0 + f.Sq)) - (int)f.q0;
  float2 sk = {0.f, 0.f}, sv = {0.f, 0.f};
  float sd = 0.f;
  if (r0 < r1) {
    const int g0 = r0 / kGroupRows, g1 = (r1 - 1) / kGroupRows;
    for (int gb = g0; gb <= g1; gb += kRedBatch) {
      int64_t o[kRedBatch];
#pragma unroll
      for (int u = 0; u < kRedBatch; ++u) {
        const int64_t gi = seg * a.n_super + min(gb + u, g1);
        // a kept key is a candidate of each of these groups; the clamp only keeps
        // the read inside the group's rows whatever the map holds
        o[u] = gi * a.cap + min(max(a.pmap[gi * f.Sk + j], 0), (int)a.cap - 1);
      }
      // every load is issued before any is used (past g1 they reread group
      // g1's row and are dropped), so the batch's loads are all in flight
      float2 x[kRedBatch], y[kRedBatch];
      float z[kRedBatch];
#pragma unroll
      for (int u = 0; u < kRedBatch; ++u) {
        x[u] = reinterpret_cast<const float2*>(a.pk + o[u] * kD)[lane];
        y[u] = reinterpret_cast<const float2*>(a.pv + o[u] * kD)[lane];
        z[u] = a.pd[o[u]];
      }
#pragma unroll
      for (int u = 0; u < kRedBatch; ++u) {
        const bool in = gb + u <= g1;
        sk.x += in ? x[u].x : 0.f;
        sk.y += in ? x[u].y : 0.f;
        sv.x += in ? y[u].x : 0.f;
        sv.y += in ? y[u].y : 0.f;
        sd += in ? z[u] : 0.f;
      }
    }
  }
  const int64_t orow = (((int64_t)b * f.Sk + j) * f.Hkv + h) * kD;
  reinterpret_cast<float2*>(a.dK + orow)[lane] = sk;
  reinterpret_cast<float2*>(a.dV + orow)[lane] = sv;
  if (lane == 0) a.ddelta[seg * f.Sk + j] = sd;
}

template <int NH>
hipError_t launch_dq(DmaBwdArgs& a, hipStream_t st) {
  const int G = (int)(a.f.Hq / a.f.Hkv);
  dim3 grid((unsigned)a.f.n_tiles, (unsigned)a.f.Hkv, (unsigned)(a.f.B * (G / NH)));
  if constexpr (NH == 4)
    hipLaunchKernelGGL(bwd_dq_pp_kernel, grid, dim3(NH * 128), 0, st, a);
  else
    hipLaunchKernelGGL(bwd_dq_kernel<NH>, grid, dim3(NH * 128), 0, st, a);
  return hipGetLastError();
}

size_t al256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

size_t dma_attn_bwd_ws_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Sk,
                             int64_t w) {
  int64_t ns = 0, cap = 0;
  dma_cand_dims(Sq, Sk, w, &ns, &cap);
  const size_t BH = (size_t)(B * Hkv);
  const size_t nt = (size_t)((Sq + kBq - 1) / kBq);
  const size_t nc = BH * (size_t)ns * (size_t)cap;
  return al256((size_t)(B * Hq * Sq) * 4) + 2 * al256(nc * 4) + al256(BH * ns * 4) +
         al256(BH * nt * 4) + 2 * al256(nc * kD * 4) + al256(nc * 4) +
         al256(BH * (size_t)ns * (size_t)Sk * 4);
}

hipError_t dma_launch_attn_bwd(DmaBwdArgs& a, hipStream_t st) {
  const DmaAttnArgs& f = a.f;
  const int64_t BH = f.B * f.Hkv;
  dma_cand_dims(f.Sq, f.Sk, f.w, &a.n_super, &a.cap);
  const size_t nt = (size_t)f.n_tiles;
  const size_t nc = (size_t)BH * (size_t)a.n_super * (size_t)a.cap;
  unsigned char* p = static_cast<unsigned char*>(f.ws);
  a.Dv = reinterpret_cast<float*>(p);
  p += al256((size_t)(f.B * f.Hq * f.Sq) * 4);
  a.cj = reinterpret_cast<int32_t*>(p);
  p += al256(nc * 4);
  a.ce = reinterpret_cast<int32_t*>(p);
  p += al256(nc * 4);
  a.ccnt = reinterpret_cast<int32_t*>(p);
  p += al256((size_t)BH * a.n_super * 4);
  a.cdmax = reinterpret_cast<float*>(p);
  p += al256((size_t)BH * nt * 4);
  a.pk = reinterpret_cast<float*>(p);
  p += al256(nc * kD * 4);
  a.pv = reinterpret_cast<float*>(p);
  p += al256(nc * kD * 4);
  a.pd = reinterpret_cast<float*>(p);
  p += al256(nc * 4);
  a.pmap = reinterpret_cast<int32_t*>(p);

  hipError_t e = dma_launch_cand(f.delta, f.evict, BH, f.Sk, f.Sq, f.q0, f.w, a.cj, a.ce, a.ccnt,
                                 a.cdmax, st);
  if (e != hipSuccess) return e;
  const int G = (int)(f.Hq / f.Hkv);
  e = G % 4 == 0 ? launch_dq<4>(a, st) : G % 2 == 0 ? launch_dq<2>(a, st) : launch_dq<1>(a, st);
  if (e != hipSuccess) return e;
  dim3 g2((unsigned)((a.cap + kSliceKeys - 1) / kSliceKeys), (unsigned)a.n_super, (unsigned)BH);
  hipLaunchKernelGGL(bwd_dkv_kernel<0>, g2, dim3(256), 0, st, a);
  hipLaunchKernelGGL(bwd_dkv_kernel<1>, g2, dim3(256), 0, st, a);
  hipLaunchKernelGGL(bwd_reduce_kernel, dim3((unsigned)((f.Sk + 3) / 4), (unsigned)BH), dim3(256),
                     0, st, a);
  return hipGetLastError();
}
