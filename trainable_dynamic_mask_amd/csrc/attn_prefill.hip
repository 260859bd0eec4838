// Masked attention of the DMA forward, bf16 prefill (Hugging Face blog
// "Trainable Dynamic Mask Sparse Attention", section "Efficient Sparse
// Attention Computation"): o = softmax(q k^T / sqrt(d) + delta) v over the keys
// the row keeps.  A masked key has weight exactly 0 ("Forward Pass Safety"),
// so its work is skipped entirely: a workgroup never visits key tiles, it
// walks the compacted list U of the keys that some row of its 64-row query
// tile keeps (built by the mask step), 64 gathered keys (one chunk) at a time.
//
// Work split: one workgroup per (query tile, kv head, batch, head group).
// Its NW = 2*NH waves are the NH query heads of one kv head (GQA) times two
// 32-row halves of the tile, so each gathered K/V chunk in LDS serves NH*64
// query rows.  Per chunk and wave:
//   S^T = K Q^T        (keys x queries) on v_mfma_f32_32x32x16_bf16, K from
//                      LDS, Q^T held in registers for the whole kernel;
//   softmax            online, base 2, per query = per lane column;
//   O^T += V^T P^T     the S^T accumulator layout is already the B operand
//                      layout, so P never moves; V is read from LDS with the
//                      transposing ds_read_b64_tr_b16.
//
// Ping-pong: the waves form two groups, A (waves 0..NW/2-1) and B (the rest),
// one wave of each per SIMD.  Each wave alternates an MFMA phase
//   G_c = { O += V(c-1) P(c-1)^T ;  S(c) = K(c) Q^T }
// and a VALU phase
//   S_c = { softmax of S(c) -> P(c) }.
// Step c ends with a workgroup barrier; in it group A runs G_c then S_c and
// group B runs S_{c-1} then G_c, so one wave of every SIMD mostly runs MFMAs
// while the other runs the softmax.
//
// Memory pipeline: K/V tiles are triple-buffered and gathered straight from
// HBM into LDS (direct loads, no registers) by the group-A waves, two steps
// before they are read; a step's loads are spread over the issuing phase so
// that the address unit is never flooded.  The key
// metadata (list entries, delta, eviction rows) moves the same way, five
// and three steps ahead, and is turned into the mask and bias of a chunk one
// step ahead.  The direct loads are inline asm, invisible to the compiler:
// every wait for them is an explicit vmcnt count at a phase barrier, and no
// wave ever consumes a register loaded from global memory inside the loop,
// so the compiler inserts no waits of its own that would stall on them.
//
// Workgroups are mapped so that each XCD (with its own L2) serves few kv
// heads, longest query tiles first.
//
// Numerics: scores are s = scale*(q.k) + delta.  delta can reach 1e4, where
// fp32 spacing is ~1e-3, so the bias enters as (delta - dmax) * log2(e) with
// dmax the largest delta of the tile's list: the subtraction is exact for
// every key within a factor 2 of dmax (the only keys with weight), and the
// constant cancels in the softmax and is added back to the log-sum-exp.  The
// bias, divided by the score scale, is the initial value of the score
// accumulator, so the MFMAs add q.k to it.
#include "lds_dma.h"

namespace {

constexpr int kBq = 64;
constexpr int kBk = 64;
constexpr int kD = 128;
// K and V tiles: 64 rows of 256 bytes, no padding.  Each row's sixteen
// 16-byte chunks are stored permuted so that the reads below hit distinct LDS
// banks: K chunk c of row r at c ^ (r % 16) (the 16 rows of one 16-byte read
// land on 16 distinct chunks), V chunk c at c ^ 4*(r % 4) (the 4 rows of one
// transposing read land on 4 disjoint 64-byte spans).
constexpr int kRowB = kD * 2;
constexpr int kTileB = kBk * kRowB;
constexpr int kBufs = 3;   // K/V tile buffers: chunk c in buffer c % 3
constexpr int kRaw = 8;    // raw key metadata (index, delta, eviction row): chunk c in slot c % 8
constexpr int kFin = 4;    // prepared key metadata (mask, bias): chunk c in slot c % 4
constexpr int kXcds = 8;        // accelerator complex dies, each with its own L2

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazy = 8.f;  // base-2 headroom before O is rescaled (weights stay <= 2^8)
// reference of a row that has met no kept key yet: finite, so that the
// exponents of its masked (-inf) logits stay -inf
constexpr float kNoRef = -3.402823466e38f;
// largest base-2 gap from a row's first largest logit up to its reference
constexpr float kFloor = 64.f;
// largest gap between the tile's largest delta and a wave's first row's own
// largest delta that the shared tile offset serves (scores up to kRefSpan /
// scale ~ 724 in magnitude keep ~2^-14 absolute precision)
constexpr float kRefSpan = 64.f;

using dma::dma_b128;
using dma::dma_b128_s;
using dma::dma_b32;
using dma::i16x4;
using dma::lds_addr;
using dma::lds_i16x4;
using dma::to_bf16x8;
using dma::u32x2;
using dma::u32x4;

// Everything the workgroup keeps in LDS (105 KB).
struct Smem {
  unsigned char k[kBufs][kTileB];  // K tiles, rows as gathered (swizzled)
  unsigned char v[kBufs][kTileB];  // V tiles
  int jraw[kRaw][kBk];             // list entries, clamped to the list: the gather rows
  float draw[kRaw][kBk];           // delta of those keys
  int eraw[kRaw][kBk];             // their eviction rows
  int pj[kFin][kBk];               // key index for the mask (INT_MAX for padding)
  int e[kFin][kBk];                // eviction row (0 for padding)
  float bias[kFin][kBk];           // (delta - dmax) * log2(e) / score scale, -inf for padding
  float dval[kFin][kBk];           // delta itself, -inf for padding (row-reference waves)
};

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
constexpr bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 r;
  r[0] = (__bf16)lo;
  r[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, r);
}

// Gather the 64 rows of one K or V chunk into the tile at LDS address tile,
// 16 bytes per lane.  The tile is 16 pieces of 1 KB = 4 rows; wave w loads
// pieces w, w+NW, ...: lane L fills row 4*piece + L/16, stored chunk L%16,
// which holds logical chunk (L%16) ^ swz(row).  idx[t] is the key index of
// the lane's row in piece w + t*NW (see gather_rows).  2 * 16/NW loads per
// wave for a K and a V tile.
template <int NW, bool IS_V>
__device__ __forceinline__ void gather_tile(uint32_t tile, const int (&idx)[16 / NW],
                                            const unsigned char* g, uint32_t rowb, int wave,
                                            int lane) {
  const int rsub = lane >> 4, pc = lane & 15;
#pragma unroll
  for (int t = 0; t < 16 / NW; ++t) {
    const int piece = wave + t * NW;
    const int row = piece * 4 + rsub;
    const int lc = pc ^ (IS_V ? ((row & 3) << 2) : (row & 15));
    dma_b128_s(g, __umul24((uint32_t)idx[t], rowb) + lc * 16, tile + piece * 1024);
  }
}

// The i-th of the 2 * 16/NW direct loads of one batch: K pieces first, then V.
template <int NW>
__device__ __forceinline__ void gather_piece(int i, uint32_t ktile, uint32_t vtile,
                                             const int (&kidx)[16 / NW], const int (&vidx)[16 / NW],
                                             const unsigned char* kg, const unsigned char* vg,
                                             uint32_t rowb, int wave, int lane) {
  constexpr int P = 16 / NW;
  const bool is_v = i >= P;
  const int t = is_v ? i - P : i;
  const int piece = wave + t * NW;
  const int row = piece * 4 + (lane >> 4);
  const int lc = (lane & 15) ^ (is_v ? ((row & 3) << 2) : (row & 15));
  const int idx = is_v ? vidx[t] : kidx[t];
  dma_b128_s(is_v ? vg : kg, __umul24((uint32_t)idx, rowb) + lc * 16,
             (is_v ? vtile : ktile) + piece * 1024);
}

// Key indices of the rows this lane gathers for chunk ch (see gather_tile):
// positions past the list repeat its last key, whose scores are masked.
template <int NW>
__device__ __forceinline__ void gather_rows(int (&idx)[16 / NW], const Smem& sm, int ch,
                                            int wave, int lane) {
#pragma unroll
  for (int t = 0; t < 16 / NW; ++t)
    idx[t] = sm.jraw[ch % kRaw][4 * (wave + t * NW) + (lane >> 4)];
}

// Workgroup barrier at the end of a phase.  This wave's LDS accesses
// complete first; with VM >= 0, so do all but its VM most recent direct
// loads (those of its current batch), so every gather issued in the
// previous batch has landed before the barrier releases the waves that read
// it.  The empty asm statements keep the compiler from moving memory
// accesses across the barrier; no fence is used, as a fence would wait for
// every load in flight.
// Built with DMA_SAFE_SYNC (the cross-check library), every barrier waits
// for all of the wave's loads instead: the results must be bit-identical.
template <int VM>
__device__ __forceinline__ void phase_barrier() {
  static_assert(VM < 64, "vmcnt holds 6 bits");
  asm volatile("" ::: "memory");
#ifdef DMA_SAFE_SYNC
  __builtin_amdgcn_s_waitcnt(0);  // vmcnt(0) expcnt(0) lgkmcnt(0)
#else
  if constexpr (VM >= 0)
    __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4));  // vmcnt(VM) lgkmcnt(0)
  else
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));  // lgkmcnt(0) only
#endif
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Running softmax state of one wave: 32 query rows.
struct Acc {
  dma::f32x16 o[4];  // O^T: 4 blocks of 32 d x 32 queries
  float m;           // base-2 reference
  float l;           // this lane's partial row sum of the weights (the log-sum-exp)
  float lr;          // the same sum of the weights as rounded to bf16 for the PV product
  float mbest;       // base-2 bias of the row's largest kept delta (its best key's bias)
};

// V^T operands of PV k-step ks = (mb, hf) = (ks/2, ks%2) for the four d
// blocks: V^T rows d = db*32 + l32, keys mb*32 + 16*hf + 4*hi + [0,4) and
// mb*32 + 16*hf + 8 + 4*hi + [0,4), matching the keys of P^T's registers.
// V stays row-major in LDS; each transposing read serves a 16-lane group
// g = lane/16: lane r of the group addresses key row kbase + r/4, columns
// dbase + 16*(g%2) + 4*(r%4), and lane i then receives that group's 4 keys
// at d = dbase + 16*(g%2) + i.
__device__ __forceinline__ void v_operands(dma::bf16x8 (&vop)[4], const unsigned char* vt,
                                           int ks, int lane) {
  const int g = lane >> 4, r = lane & 15;
  // address-space cast of the LDS tile pointer (the instruction takes a local address)
  const __attribute__((address_space(3))) unsigned char* vbase =
      (const __attribute__((address_space(3))) unsigned char*)vt;
  // key rows k0 and k0 + 8 share k0 % 4, hence the chunk permutation
  const int k0 = (ks >> 1) * 32 + 16 * (ks & 1) + 4 * (g >> 1) + (r >> 2);
  const int swz = (k0 & 3) << 2;
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    // element d0 = db*32 + 16*(g%2) + 4*(r%4): logical chunk d0/8, byte (d0%8)*2
    const int lc = db * 4 + 2 * (g & 1) + ((r & 3) >> 1);
    const int off = ((lc ^ swz) << 4) + (r & 1) * 8;
    const i16x4 lo =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vbase + k0 * kRowB + off));
    const i16x4 up =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vbase + (k0 + 8) * kRowB + off));
    const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), up2 = __builtin_bit_cast(u32x2, up);
    const u32x4 vv = {lo2[0], lo2[1], up2[0], up2[1]};
    vop[db] = __builtin_bit_cast(dma::bf16x8, vv);
  }
}

// MFMA phase G_c: S^T(c) = K(c) Q^T (rows = the chunk's 64 keys in two
// blocks of 32, cols = the wave's 32 queries; lane (l32, hi) reads K row
// mb*32 + l32, d = kk*16 + 8*hi + [0, 8)), then O^T += V(c-1)^T P(c-1)^T.
// LDS operand reads run ahead of their MFMAs: K reads four operands ahead,
// V one PV k-step ahead, so the matrix cores do not wait on single LDS
// reads.  The sched_group_barrier sequence pins that order (0x100 = LDS
// read, 0x008 = MFMA) and bounds the registers held by operands in flight.
template <int NDMA, bool ROWREF, typename F>
__device__ __forceinline__ void g_phase(Acc& acc, const dma::bf16x8 (&pb)[2][2],
                                        dma::f32x16 (&s)[2], const dma::bf16x8 (&qf)[8],
                                        const unsigned char* kt, const unsigned char* vt,
                                        const float* bias_row, const float* dval_row,
                                        float rref, float bias_div, int lane, F&& dma_issue) {
  const int l32 = lane & 31, hi = lane >> 5;
  // Both waves of a SIMD keep the same issue priority: with one barrier per
  // step, raising this phase's wave measured 1.9% slower at 16K (it delays
  // the softmax wave sharing the SIMD, which then ends the step late).
  // the scores start from the keys' bias divided by the score scale, so the
  // MFMAs add q.k to it (register i of block mb holds key mb*32 + 8*(i/4) +
  // 4*hi + i%4; the rows point at key 4*hi of the chunk).  Waves whose rows
  // take their own reference (ROWREF) form the bias from delta and the
  // lane's row reference: all 32 values of a lane belong to one query row.
  if constexpr (ROWREF) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 dv = *reinterpret_cast<const float4*>(dval_row + mb * 32 + 8 * q4);
        s[mb][4 * q4 + 0] = (dv.x - rref) * bias_div;
        s[mb][4 * q4 + 1] = (dv.y - rref) * bias_div;
        s[mb][4 * q4 + 2] = (dv.z - rref) * bias_div;
        s[mb][4 * q4 + 3] = (dv.w - rref) * bias_div;
      }
  } else {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 bv = *reinterpret_cast<const float4*>(bias_row + mb * 32 + 8 * q4);
        s[mb][4 * q4 + 0] = bv.x;
        s[mb][4 * q4 + 1] = bv.y;
        s[mb][4 * q4 + 2] = bv.z;
        s[mb][4 * q4 + 3] = bv.w;
      }
  }
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    // the direct loads handed to this phase go out evenly between the score
    // MFMAs, so the address unit is never flooded and the wave never stalls
    // on a full load queue
    if constexpr (NDMA > 0) {
      constexpr int kEvery = NDMA >= 16 ? 1 : 16 / NDMA;
      if (q % kEvery == 0) {
#pragma unroll
        for (int i = 0; i < (NDMA + 15) / 16; ++i) dma_issue((q / kEvery) * ((NDMA + 15) / 16) + i);
      }
    }
    const int kk = q >> 1, mb = q & 1;
    const int row = mb * 32 + l32;
    const dma::bf16x8 kop = *reinterpret_cast<const dma::bf16x8*>(
        kt + row * kRowB + (((kk * 2 + hi) ^ (row & 15)) << 4));
    s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qf[kk], s[mb], 0, 0, 0);
  }
  dma::bf16x8 va[4], vb[4];
  v_operands(va, vt, 0, lane);
  v_operands(vb, vt, 1, lane);
#pragma unroll
  for (int db = 0; db < 4; ++db)
    acc.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[db], pb[0][0], acc.o[db], 0, 0, 0);
  v_operands(va, vt, 2, lane);
#pragma unroll
  for (int db = 0; db < 4; ++db)
    acc.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vb[db], pb[0][1], acc.o[db], 0, 0, 0);
  v_operands(vb, vt, 3, lane);
#pragma unroll
  for (int db = 0; db < 4; ++db)
    acc.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[db], pb[1][0], acc.o[db], 0, 0, 0);
#pragma unroll
  for (int db = 0; db < 4; ++db)
    acc.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vb[db], pb[1][1], acc.o[db], 0, 0, 0);
  // order: bias reads, K reads 4 ahead of the 16 score MFMAs, V k-step 0
  // read during the last 4 of them, then each PV k-step after the reads of
  // the next one
  __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);
#pragma unroll
  for (int q = 0; q < 12; ++q) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
#pragma unroll
  for (int ks = 0; ks < 3; ++ks) {
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
}

// Weights of one chunk as the bf16 B operands of the PV product, and their
// sums.  FIRST: the scores s become the exponents x = scale2*s - m in place
// (x = s - m when ROUNDED: s is the rounded logit) and P = exp2(x); otherwise
// s already holds exponents and P = exp2(s - m).  O is normalised by the sum
// of the weights exactly as the PV product sees them (rounded to bf16): then
// a row dominated by one key returns that key's value row with no error from
// the weight's rounding.  The sum of rounded pairs is one bf16 dot product
// with (1, 1) per two weights.  The log-sum-exp (ROUNDED: asked for) uses the
// unrounded weights.  Four partial sums keep the dependency chains short.
// The group's direct loads (NDMA per phase) go out evenly over the pass.
template <bool ROUNDED, bool FIRST, int NDMA, typename F>
__device__ __forceinline__ void weights_pass(dma::f32x16 (&s)[2], dma::bf16x8 (&pb)[2][2],
                                             float m_use, float scale2, float& sum_p,
                                             float& sum_r, F&& dma_issue) {
  float rsp[4] = {0.f, 0.f, 0.f, 0.f};
  float rsr[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      if constexpr (NDMA > 0) {
#pragma unroll
        for (int i = 0; i < NDMA / 4; ++i) dma_issue((mb * 2 + hf) * (NDMA / 4) + i);
      }
      float p[8];
#pragma unroll
      for (int t8 = 0; t8 < 8; ++t8) {
        const int i = hf * 8 + t8;
        if constexpr (FIRST) {
          s[mb][i] = ROUNDED ? s[mb][i] - m_use : fmaf(s[mb][i], scale2, -m_use);
          p[t8] = __builtin_amdgcn_exp2f(s[mb][i]);
        } else {
          p[t8] = __builtin_amdgcn_exp2f(s[mb][i] - m_use);
        }
        if constexpr (ROUNDED) rsp[t8 & 3] += p[t8];
      }
      pb[mb][hf] = to_bf16x8(p);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const bf16x2 pr = {pb[mb][hf][2 * k], pb[mb][hf][2 * k + 1]};
        rsr[k] = __builtin_amdgcn_fdot2_f32_bf16(pr, kOnes2, rsr[k], false);
      }
    }
  if constexpr (ROUNDED) sum_p = (rsp[0] + rsp[1]) + (rsp[2] + rsp[3]);
  sum_r = (rsr[0] + rsr[1]) + (rsr[2] + rsr[3]);
}

// Rescale of O and the sums when a row's reference m grows by d >= 0.
__device__ __forceinline__ void rescale(Acc& acc, float d) {
  const float alpha = __builtin_amdgcn_exp2f(-d);
  acc.l *= alpha;
  acc.lr *= alpha;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc.o[db][i] *= alpha;
  acc.m += d;
}

// Largest of x over the two lanes of one query (lane and lane ^ 32), by the
// gfx950 lane swap between the wave's halves (no LDS round trip).
__device__ __forceinline__ float row_max2(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                   false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}

// Largest of the lane's 32 values.
__device__ __forceinline__ float lane_max(const dma::f32x16 (&s)[2]) {
  float mxp[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) mxp[i & 3] = fmaxf(mxp[i & 3], s[mb][i]);
  return fmaxf(fmaxf(mxp[0], mxp[1]), fmaxf(mxp[2], mxp[3]));
}

// Softmax of one chunk: logits in the base-2 domain, lazy rescale of O, and
// the weights P.  MASKED chunks hold keys that only some rows of the tile
// keep and apply j <= p < e_j per element; the others hold keys every row
// keeps.  Lane (l32, hi) holds key(mb, i) = mb*32 + 8*(i/4) + 4*hi + i%4 of
// query l32; the other 32 keys of the same query sit in lane ^ 32.
//
// The lazy rule: a row's reference m moves only when one of its logits
// exceeds it by more than kLazy, and then every lane of the wave moves m to
// the largest logit of its query (both halves) and rescales O.  Such a logit
// has a weight above 2^kLazy, which rounds to at least 2^kLazy in bf16, so
// the lane's sum of the rounded weights (needed anyway) reaches 2^kLazy.
// Hence, once every row of the wave has a reference, the common path takes
// no maximum: the weights are computed against the current m, and only when
// some lane's sum reaches 2^kLazy (a NaN sum counts) does the wave take the
// maximum of the exponents, apply the rule and, if it fired, recompute the
// weights from the exponents kept in place.  A row's first reference comes
// from its first kept keys and the bias of its best key (below), so that the
// rule fires only on unusually large score terms (or where delta is heavy-
// tailed and a row's first keys lie far below its best one).
template <bool MASKED, bool ROUNDED, int NDMA, typename F>
__device__ __forceinline__ void softmax_phase(Acc& acc, dma::f32x16 (&s)[2],
                                              dma::bf16x8 (&pb)[2][2], const Smem& sm, int slot,
                                              int hi, int pos, float scale2, F&& dma_issue) {
  if constexpr (MASKED || ROUNDED) {
    const int* pjp = &sm.pj[slot][4 * hi];
    const int* pep = &sm.e[slot][4 * hi];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int kb = mb * 32 + 8 * q4;
        int4 jv = {0, 0, 0, 0}, evv = {0, 0, 0, 0};
        if constexpr (MASKED) {
          jv = *reinterpret_cast<const int4*>(pjp + kb);
          evv = *reinterpret_cast<const int4*>(pep + kb);
        }
        const int pj[4] = {jv.x, jv.y, jv.z, jv.w};
        const int pe[4] = {evv.x, evv.y, evv.z, evv.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = q4 * 4 + r;
          // the logit is scale2 * v with v = q.k + bias / scale2.  ROUNDED
          // rounds it first, as the backward recomputes it; otherwise the
          // factor goes into the exponent
          float v = ROUNDED ? s[mb][i] * scale2 : s[mb][i];
          // kept iff pj <= pos < pe, one unsigned compare (pe <= pj: never)
          if constexpr (MASKED)
            v = ((uint32_t)(pos - pj[r]) < (uint32_t)(pe[r] - pj[r])) ? v : -INFINITY;
          s[mb][i] = v;
        }
      }
  }
  constexpr float kLazyW = 256.f;  // 2^kLazy
  static_assert(kLazy == 8.f, "kLazyW is 2^kLazy");
  if (__ballot(acc.m == kNoRef) != 0ull) {
    // A row with no reference yet (O and the sums still 0) that has kept
    // keys in this chunk takes the larger of their largest logit c and the
    // bias mbest of its best key, but at most c + kFloor: later keys then only
    // exceed the reference by more than kLazy when their score term
    // (q.k)*scale*log2(e) does, and the row's largest weight stays at least
    // 2^-kFloor.  Rows that have a reference keep it.
    float mx = lane_max(s);
    if constexpr (!ROUNDED) mx *= scale2;  // scale2 > 0 keeps the maximum
    mx = row_max2(mx);
    if (acc.m == kNoRef && mx > -INFINITY) acc.m = fminf(fmaxf(mx, acc.mbest), mx + kFloor);
  }
  float sum_p = 0.f, sum_r;
  // rows still without a reference have every logit at -inf: weights 0
  weights_pass<ROUNDED, true, NDMA>(s, pb, acc.m, scale2, sum_p, sum_r, dma_issue);
  if (__ballot(!(sum_r < kLazyW)) != 0ull) {
    // s holds the exponents x = logit - m now; the row's largest logit so far
    // is m + (largest x of both halves)
    const float mx = lane_max(s);
    if (__ballot(mx > kLazy) != 0ull) {
      const float d = fmaxf(row_max2(mx), 0.f);
      rescale(acc, d);
      weights_pass<ROUNDED, false, 0>(s, pb, d, scale2, sum_p, sum_r, [](int) {});
    }
  }
  if constexpr (ROUNDED) acc.l += sum_p;
  acc.lr += sum_r;
}

template <int NH, bool ROUNDED>
__global__ __launch_bounds__(NH * 128, 1) void attn_prefill_bf16_kernel(DmaAttnArgs a) {
  constexpr int NW = NH * 2;
  constexpr int NG = 2 * (16 / NW);  // direct loads per wave for one K and one V tile
  // In the chunk loop one group-A wave issues the key metadata loads and
  // another prepares the mask and bias: with four waves per group these are
  // waves 1 and 3, whose softmax phase ends earliest (wave 0 and 2 had ~900
  // cycles per step less slack when measured).
  constexpr int kLoadWave = NW >= 4 ? 1 : 0;
  constexpr int kPrepWave = NW >= 8 ? 3 : 0;
  __shared__ __align__(16) Smem sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int G = (int)(a.Hq / a.Hkv);
  const int ngrp = G / NH;
  // Workgroups are dealt to the 8 XCDs round-robin by linear id.  When the
  // (batch, kv head, head group) combinations split evenly over the XCDs,
  // XCD x takes combinations x, x+8, ... whole, so each L2 holds the K/V rows
  // of few heads; within a combination the longest tiles (last) go first.
  const int ntile = (int)a.n_tiles;
  const int ncomb = (int)(a.B * a.Hkv) * ngrp;
  const int lid = blockIdx.x;
  int t, comb;
  if (ncomb % kXcds == 0) {
    const int xcd = lid % kXcds, slot = lid / kXcds;
    comb = (slot / ntile) * kXcds + xcd;
    t = ntile - 1 - slot % ntile;
  } else {
    comb = lid / ntile;
    t = ntile - 1 - lid % ntile;
  }
  const int hgrp = comb % ngrp;
  const int h = (comb / ngrp) % (int)a.Hkv;
  const int b = comb / (ngrp * (int)a.Hkv);
  const int hq = h * G + hgrp * NH + (wave >> 1);
  const int half = wave & 1;
  const bool grp_a = wave < NW / 2;
  const int64_t seg = (int64_t)b * a.Hkv + h;
  const int64_t g = seg * a.n_tiles + t;
  const int r_lo = t * kBq;
  const int rows = min(kBq, (int)a.Sq - r_lo);
  const int p_lo = (int)a.q0 + r_lo;
  const int cnt = a.u_cnt[g];
  const int nfull = a.u_nfull[g];
  const float dmax = a.u_dmax[g];
  const int32_t* list = a.u_idx + g * a.u_stride;
  const float* dl = a.delta + seg * a.Sk;
  const int32_t* ev = a.evict + seg * a.Sk;
  const int nch = (cnt + kBk - 1) / kBk;
  const int nplain = nfull / kBk;  // leading chunks that every row keeps whole
  const unsigned char* Kg =
      static_cast<const unsigned char*>(a.K) + (b * a.ksb + h * a.ksh) * 2;
  const unsigned char* Vg =
      static_cast<const unsigned char*>(a.V) + (b * a.ksb + h * a.ksh) * 2;
  // row stride in bytes; the host checks that offsets fit 32 bits and that
  // key indices and the stride fit 24 (the row offsets use the full-rate
  // 24-bit multiply)
  const uint32_t rowb = (uint32_t)(a.kss * 2);
  const float scale2 = a.scale * kLog2e;
  const float bias_div = kLog2e / scale2;  // bias enters the scores before the scale
  const uint32_t lds_k = lds_addr(&sm.k[0][0]), lds_v = lds_addr(&sm.v[0][0]);
  const uint32_t lds_j = lds_addr(&sm.jraw[0][0]), lds_d = lds_addr(&sm.draw[0][0]),
                 lds_e = lds_addr(&sm.eraw[0][0]);
  const int clast = max(cnt - 1, 0);

  // Q^T operand: lane holds query n = half*32 + l32, d = kk*16 + 8*hi + [0, 8)
  const int n = half * 32 + l32;
  const int pos = p_lo + n;
  // Row reference.  Row p keeps its best key, so its largest kept delta is
  // the prefix maximum r(p) of delta over keys 0..p: the largest delta before
  // the tile (from the mask step), then the running maximum over the tile's
  // own keys p_lo..p.  A wave whose first row's r lies far below the tile's
  // dmax (a key with a much larger delta is born later in the tile) offsets
  // its scores by each row's own r instead of dmax, so the scores it carries
  // stay small and keep their precision.
  float rref = (lane < rows) ? dl[p_lo + lane] : -INFINITY;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float y = __shfl_up(rref, o);
    if (lane >= o) rref = fmaxf(rref, y);
  }
  rref = fmaxf(a.u_dlo[g], __shfl(rref, n));
  const float rfirst = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(rref)));
  const bool rowref = rfirst > -INFINITY && dmax - rfirst > kRefSpan;
  dma::bf16x8 qf[8];
  {
    const uint16_t* qrow = static_cast<const uint16_t*>(a.Q) + b * a.qsb + hq * a.qsh +
                           (int64_t)(r_lo + (n < rows ? n : 0)) * a.qss;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      // rows past the tile's end repeat its first row; their output is not written
      const u32x4 v = *reinterpret_cast<const u32x4*>(qrow + kk * 16 + hi * 8);
      qf[kk] = __builtin_bit_cast(dma::bf16x8, v);
    }
  }

  // Key metadata (wave 0 in the prologue, kLoadWave and kPrepWave in the
  // loop): the list entries of chunk x are loaded straight into slot x % 8
  // of jraw five steps before chunk x is first multiplied, delta and the
  // eviction rows of those keys three steps before (addressed by the landed
  // list entries), and in the step before, they become the mask and bias of
  // slot x % 4, with the positions past the list padded.
#define DMA_LIST(x_) dma_b32(list + min((x_) * kBk + lane, clast), lds_j + ((x_) % kRaw) * 256)
#define DMA_DELTA(x_, j_)                                   \
  do {                                                      \
    dma_b32(dl + (j_), lds_d + ((x_) % kRaw) * 256);        \
    dma_b32(ev + (j_), lds_e + ((x_) % kRaw) * 256);        \
  } while (0)
#define DMA_PREPARE(x_)                                                         \
  do {                                                                          \
    const int sr_ = (x_) % kRaw, sf_ = (x_) % kFin;                             \
    const bool pad_ = (x_) * kBk + lane >= cnt;                                 \
    const int jj_ = sm.jraw[sr_][lane];                                         \
    sm.pj[sf_][lane] = pad_ ? 0x7fffffff : jj_;                                 \
    sm.e[sf_][lane] = pad_ ? 0 : sm.eraw[sr_][lane];                            \
    sm.bias[sf_][lane] = pad_ ? -INFINITY : (sm.draw[sr_][lane] - dmax) * bias_div; \
    sm.dval[sf_][lane] = pad_ ? -INFINITY : sm.draw[sr_][lane];                 \
  } while (0)

  // prologue: list entries of chunks 0..4, then delta of chunks 0..2
  // together with K(0), then the mask and bias of chunk 0; every load of it
  // has landed when it ends (two load latencies in a row)
  if (wave == 0) {
#pragma unroll
    for (int x = 0; x < 5; ++x) DMA_LIST(x);
  }
  for (int i = tid; i < kTileB / 16; i += NW * 64)  // V(-1) = 0 (buffer 2)
    reinterpret_cast<u32x4*>(sm.v[2])[i] = u32x4{0u, 0u, 0u, 0u};
  if (wave == 0) {
    __builtin_amdgcn_s_waitcnt(7 << 4);  // vmcnt(0): the list entries have landed
    asm volatile("" ::: "memory");
#pragma unroll
    for (int x = 0; x < 3; ++x) {
      const int jj = sm.jraw[x][lane];
      DMA_DELTA(x, jj);
    }
  }
  phase_barrier<-1>();  // the list entries are visible; delta is still in flight
  // K(0) -> buffer 0, and already K(1) -> 1 and V(0) -> 0, all in flight together
  {
    int pk[16 / NW], pv[16 / NW];
    gather_rows<NW>(pk, sm, 0, wave, lane);
    gather_tile<NW, false>(lds_k, pk, Kg, rowb, wave, lane);
    gather_rows<NW>(pk, sm, 1, wave, lane);
    gather_rows<NW>(pv, sm, 0, wave, lane);
    gather_tile<NW, false>(lds_k + 1 * kTileB, pk, Kg, rowb, wave, lane);
    gather_tile<NW, true>(lds_v + 0 * kTileB, pv, Vg, rowb, wave, lane);
  }
  int kr[16 / (NW / 2)], vr[16 / (NW / 2)];
  __builtin_amdgcn_s_waitcnt(7 << 4);  // vmcnt(0)
  asm volatile("" ::: "memory");
  if (wave == 0) DMA_PREPARE(0);
  phase_barrier<0>();

  Acc acc;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc.o[db][i] = 0.f;
  acc.m = kNoRef;
  // Every kept delta of row p is at most r(p), which one kept key reaches,
  // so the row's logits lie below mbest + (q.k)*scale*log2(e), and one of
  // them is at least mbest - |q.k|*scale*log2(e).
  acc.mbest = rowref ? 0.f : (rref - dmax) * kLog2e;
  acc.l = 0.f;
  acc.lr = 0.f;
  dma::f32x16 s[2];
  // P(-1) = 0 against a zeroed V buffer: the PV half of G_0 adds nothing
  dma::bf16x8 pb[2][2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int t8 = 0; t8 < 8; ++t8) pb[mb][hf][t8] = (__bf16)0.f;

  // One workgroup barrier per step.  In step c group A runs G_c then S_c,
  // group B runs S_{c-1} then G_c, so while one wave of a SIMD multiplies the
  // other mostly exponentiates, and within the step the two halves may slide
  // against each other (a barrier between the two phases as well cost 16% in
  // a replica of the loop).  G_c reads K(c) from buffer c%3 and V(c-1) from
  // buffer (c+2)%3.  In step c the group-A waves gather K(c+2) into buffer
  // (c+2)%3 and V(c+1) into buffer (c+1)%3, both last read in step c-1,
  // spread over their softmax phase S_c (group B's softmax, which overlaps
  // group A's MFMA phase, ends the step; group A's has slack, and moving the
  // loads there measured 1.5% faster than half of them in each group).  At
  // the barrier ending step c a group-A wave waits for all its loads but
  // those of step c, so the tiles read in step c+1 have landed.  kLoadWave adds three metadata loads
  // per step (list entries five steps ahead, delta and eviction rows three
  // ahead); kPrepWave prepares the mask and bias of chunk c+1, into a slot
  // that no one reads in step c, from raw metadata whose loads its issuer
  // waited for before the barrier that ended step c-1.  Both groups pass
  // nch + 1 barriers in the loop; step nch of group A and step 0 of group B
  // have no softmax, G_0 multiplies the zero P(-1) by the zeroed V(-1), and
  // the scores of G_nch (padding keys) are unused.
#define DMA_TILES(c_)                                                 \
  const int b0_ = (c_) % kBufs;                                       \
  const int b2_ = b0_ == 0 ? 2 : b0_ - 1; /* (c+2) % 3 */              \
  const unsigned char* KC = sm.k[b0_];                                \
  const unsigned char* VP = sm.v[b2_]
#define DMA_STEP_A(MASKED, RR)                                                          \
  do {                                                                                  \
    DMA_TILES(c);                                                                       \
    const int b1_ = b0_ == 2 ? 0 : b0_ + 1; /* (c+1) % 3 */                             \
    const uint32_t kt_ = lds_k + b2_ * kTileB, vt_ = lds_v + b1_ * kTileB;              \
    int jd = 0;                                                                         \
    if (wave == kLoadWave) jd = sm.jraw[(c + 3) % kRaw][lane];                          \
    g_phase<0, RR>(acc, pb, s, qf, KC, VP, &sm.bias[c % kFin][4 * hi],                  \
                   &sm.dval[c % kFin][4 * hi], rref, bias_div, lane, [](int) {});           \
    asm volatile("" ::: "memory"); __builtin_amdgcn_sched_barrier(0);                    \
    if (wave == kLoadWave) {                                                            \
      DMA_LIST(c + 5);                                                                  \
      DMA_DELTA(c + 3, jd);                                                             \
    }                                                                                   \
    if (wave == kPrepWave) DMA_PREPARE(c + 1);                                          \
    asm volatile("" ::: "memory"); __builtin_amdgcn_sched_barrier(0);                    \
    if (c < nch)                                                                        \
      softmax_phase<MASKED, ROUNDED, 2 * NG>(acc, s, pb, sm, c % kFin, hi, pos, scale2,  \
                                             [&](int i_) {                              \
        gather_piece<NW / 2>(i_, kt_, vt_, kr, vr, Kg, Vg, rowb, wave, lane);           \
      });                                                                               \
    gather_rows<NW / 2>(kr, sm, c + 3, wave, lane);                                     \
    gather_rows<NW / 2>(vr, sm, c + 2, wave, lane);                                     \
    if (wave == kLoadWave)                                                              \
      phase_barrier<2 * NG + 3>();                                                      \
    else                                                                                \
      phase_barrier<2 * NG>();                                                          \
  } while (0)
#define DMA_STEP_B(MASKED, RR)                                                          \
  do {                                                                                  \
    DMA_TILES(c);                                                                       \
    g_phase<0, RR>(acc, pb, s, qf, KC, VP, &sm.bias[c % kFin][4 * hi],                  \
                   &sm.dval[c % kFin][4 * hi], rref, bias_div, lane, [](int) {});           \
    phase_barrier<-1>();                                                                \
    if (c < nch)                                                                        \
      softmax_phase<MASKED, ROUNDED, 0>(acc, s, pb, sm, c % kFin, hi, pos, scale2, [](int) {});  \
  } while (0)

  // Chunks [0, nplain) hold only keys every row keeps; the rest need the
  // per-element mask; separate loops keep the two bodies' registers apart.
  // Group B's loop body is its step's second half (G_c) followed by the
  // first half of the next step (S_c).
  int c = 0;
  if (grp_a) {
    gather_rows<NW / 2>(kr, sm, 2, wave, lane);
    gather_rows<NW / 2>(vr, sm, 1, wave, lane);
    if (rowref) {  // a separate copy of the loops keeps the common one unchanged
      for (; c < nplain; ++c) DMA_STEP_A(false, true);
      for (; c <= nch; ++c) DMA_STEP_A(true, true);
    } else {
      for (; c < nplain; ++c) DMA_STEP_A(false, false);
      for (; c <= nch; ++c) DMA_STEP_A(true, false);
    }
  } else {
    if (rowref) {
      for (; c < nplain; ++c) DMA_STEP_B(false, true);
      for (; c <= nch; ++c) DMA_STEP_B(true, true);
    } else {
      for (; c < nplain; ++c) DMA_STEP_B(false, false);
      for (; c <= nch; ++c) DMA_STEP_B(true, false);
    }
  }
  // no direct load may still be writing LDS when the workgroup ends
  __builtin_amdgcn_s_waitcnt(7 << 4);
#undef DMA_STEP_A
#undef DMA_STEP_B
#undef DMA_TILES
#undef DMA_PREPARE
#undef DMA_DELTA
#undef DMA_LIST

  // epilogue: normalise and write O (and the log-sum-exp)
  const float lt = acc.l + __shfl_xor(acc.l, 32);
  const float ltr = acc.lr + __shfl_xor(acc.lr, 32);
  const float inv = ltr > 0.f ? 1.f / ltr : 0.f;
  // O goes out through LDS so that each store instruction writes whole
  // 256-byte rows: the wave's 32 x 128 bf16 tile is written to its own LDS
  // region (rows padded to 272 bytes) in the accumulator layout, then read
  // back and stored 16 bytes per lane, 16 lanes per row.  The K/V buffers
  // are free once every wave's direct loads have landed.
  __syncthreads();
  constexpr int kOutRowB = kRowB + 16;
  static_assert(8 * 32 * kOutRowB <= (int)(sizeof(sm.k) + sizeof(sm.v)), "O staging fits");
  unsigned char* ow = &sm.k[0][0] + wave * (32 * kOutRowB);
  auto wave_sync = [] {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  // one bf16 [32 x 128] tile of the wave (O, then its rounding residual)
  // from LDS to rows of dst
  auto store_rows = [&](uint16_t* dst) {
    wave_sync();
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int r = it * 4 + (lane >> 4);  // the wave's row r: query half*32 + r
      const u32x4 v = *reinterpret_cast<const u32x4*>(ow + r * kOutRowB + (lane & 15) * 16);
      if (half * 32 + r < rows)
        *reinterpret_cast<u32x4*>(dst + (((int64_t)b * a.Sq + r_lo + half * 32 + r) * a.Hq + hq) * kD +
                                  (lane & 15) * 8) = v;
    }
    wave_sync();
  };
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d = db * 32 + 8 * q4 + 4 * hi;
      u32x2 u;
      u[0] = pack_bf16x2(acc.o[db][q4 * 4 + 0] * inv, acc.o[db][q4 * 4 + 1] * inv);
      u[1] = pack_bf16x2(acc.o[db][q4 * 4 + 2] * inv, acc.o[db][q4 * 4 + 3] * inv);
      *reinterpret_cast<u32x2*>(ow + l32 * kOutRowB + d * 2) = u;
    }
  store_rows(static_cast<uint16_t*>(a.O));
  if (a.ores) {
    // x - bf16(x) is exact in fp32; stored in bf16 it carries x to ~2^-18
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = db * 32 + 8 * q4 + 4 * hi;
        float x[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) x[k] = acc.o[db][q4 * 4 + k] * inv;
        const uint32_t u0 = pack_bf16x2(x[0], x[1]), u1 = pack_bf16x2(x[2], x[3]);
        u32x2 r;
        r[0] = pack_bf16x2(x[0] - dma::bf16_lo(u0), x[1] - dma::bf16_hi(u0));
        r[1] = pack_bf16x2(x[2] - dma::bf16_lo(u1), x[3] - dma::bf16_hi(u1));
        *reinterpret_cast<u32x2*>(ow + l32 * kOutRowB + d * 2) = r;
      }
    store_rows(static_cast<uint16_t*>(a.ores));
  }
  if (n < rows) {
    if (a.lse && hi == 0)
      a.lse[((int64_t)b * a.Hq + hq) * a.Sq + r_lo + n] =
          (acc.m + __log2f(lt)) * kLn2 + (rowref ? rref : dmax);
  }
}

template <int NH>
hipError_t launch(const DmaAttnArgs& a, hipStream_t st) {
  const int G = (int)(a.Hq / a.Hkv);
  dim3 grid((unsigned)(a.n_tiles * a.Hkv * a.B * (G / NH)));
  // With the log-sum-exp requested (the statistic a backward consumes) the
  // logits are rounded exactly as the backward recomputes them: in rows
  // whose softmax is nearly one-hot the gradients are differences of nearly
  // equal terms, and this keeps the forward's weights and lse consistent with
  // the backward's to the last bit there.  Without it the score scale is
  // applied inside the exponent (one fused multiply-add per score).
  if (a.lse)
    hipLaunchKernelGGL((attn_prefill_bf16_kernel<NH, true>), grid, dim3(NH * 128), 0, st, a);
  else
    hipLaunchKernelGGL((attn_prefill_bf16_kernel<NH, false>), grid, dim3(NH * 128), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t dma_launch_attn_prefill_bf16(const DmaAttnArgs& a, hipStream_t st) {
  const int G = (int)(a.Hq / a.Hkv);
  if (G % 4 == 0) return launch<4>(a, st);
  if (G % 2 == 0) return launch<2>(a, st);
  return launch<1>(a, st);
}
