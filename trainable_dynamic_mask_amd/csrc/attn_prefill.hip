// Masked attention of the DMA forward, bf16 prefill (Hugging Face blog
// "Trainable Dynamic Mask Sparse Attention", section "Efficient Sparse
// Attention Computation"): o = softmax(q k^T / sqrt(d) + delta) v over the keys
// the row keeps.  A masked key has weight exactly 0 ("Forward Pass Safety"),
// so its work is skipped entirely: a workgroup never visits key tiles, it
// walks the compacted list U of the keys that some row of its 64-row query
// tile keeps (built by the mask step), 64 gathered keys at a time.
//
// Work split: one workgroup per (query tile, kv head, batch, head group).
// Its NW waves are NW query heads of the same kv head (GQA), so each gathered
// K/V chunk in LDS serves NW*64 query rows.  Per chunk and wave:
//   S^T = K Q^T        (keys x queries) on v_mfma_f32_32x32x16_bf16, K from
//                      LDS, Q^T held in registers for the whole kernel;
//   online softmax     in the base-2 domain, per query = per lane column;
//   O^T += V^T P^T     the S^T accumulator layout is already the B operand
//                      layout, so P never moves; V is stored transposed in
//                      LDS ([d][key]) so the A operand is two 8-byte reads.
// Chunks are double-buffered: the gather of chunk c+1 and the key metadata
// of chunk c+2 are in flight while chunk c is computed.
//
// Numerics: scores are s = scale*(q.k) + delta.  delta can reach 1e4, where
// fp32 spacing is ~1e-3, so the bias enters as (delta - dmax) * log2(e) with
// dmax the largest delta of the tile's list: the subtraction is exact for
// every key within a factor 2 of dmax (the only keys with weight), and the
// constant cancels in the softmax and is added back to the log-sum-exp.
#include "common.h"

namespace {

constexpr int kBq = 64;
constexpr int kBk = 64;
constexpr int kD = 128;
constexpr int kKRow = kD + 8;   // K tile row, bf16 elements (272 bytes: spreads LDS banks)
// V tile row: 320 bytes, so the 8 rows x 64 bytes of one transposing read fall
// on distinct banks (64- or 32-bank LDS) and the 16-byte row stores stay
// conflict free.
constexpr int kVRow = kD + 32;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazy = 8.f;  // base-2 headroom before O is rescaled (weights stay <= 2^8)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// K/V tiles are double-buffered (chunk c in buffer c%2); key metadata uses
// three slots (chunk c in slot c%3) because it is written two chunks ahead.
struct Smem {
  uint16_t k[2][kBk * kKRow];
  uint16_t v[2][kBk * kVRow];   // V rows as gathered (read transposed, see PV below)
  int j[3][kBk];       // key index per chunk slot (gather addresses)
  int e[3][kBk];       // eviction row per slot
  int pj[3][kBk];      // key index per slot for the mask (INT_MAX for padding)
  float bias[3][kBk];  // (delta - dmax) * log2(e), -inf for padding
};

__device__ __forceinline__ dma::bf16x8 to_bf16x8(const float (&p)[8]) {
  dma::bf16x8 r;
#pragma unroll
  for (int t = 0; t < 8; ++t) r[t] = (__bf16)p[t];  // v_cvt_pk_bf16_f32, round to nearest even
  return r;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 r;
  r[0] = (__bf16)lo;
  r[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, r);
}

// Register staging of one gathered chunk.  Thread tid owns units
// u = tid + k*NT of (key pair, 16-byte d-chunk); 16 consecutive threads read
// one 256-byte key row.  K and V rows are stored as read.
template <int NT>
struct Stage {
  static constexpr int kUnits = (kBk / 2) * (kD / 8) / NT;
  u32x4 k[kUnits][2], v[kUnits][2];

  __device__ __forceinline__ void gather(const int* js, const uint16_t* Kg, const uint16_t* Vg,
                                         int64_t kss, int tid) {
#pragma unroll
    for (int u = 0; u < kUnits; ++u) {
      const int pr = tid + u * NT;
      const int kp = pr >> 4, ch = pr & 15;
      const int2 jj = *reinterpret_cast<const int2*>(&js[kp * 2]);
      const int64_t o0 = (int64_t)jj.x * kss + ch * 8, o1 = (int64_t)jj.y * kss + ch * 8;
      k[u][0] = *reinterpret_cast<const u32x4*>(Kg + o0);
      k[u][1] = *reinterpret_cast<const u32x4*>(Kg + o1);
      v[u][0] = *reinterpret_cast<const u32x4*>(Vg + o0);
      v[u][1] = *reinterpret_cast<const u32x4*>(Vg + o1);
    }
  }

  __device__ __forceinline__ void store(uint16_t* ks, uint16_t* vs, int tid) const {
#pragma unroll
    for (int u = 0; u < kUnits; ++u) {
      const int pr = tid + u * NT;
      const int kp = pr >> 4, ch = pr & 15;
      *reinterpret_cast<u32x4*>(&ks[(kp * 2) * kKRow + ch * 8]) = k[u][0];
      *reinterpret_cast<u32x4*>(&ks[(kp * 2 + 1) * kKRow + ch * 8]) = k[u][1];
      *reinterpret_cast<u32x4*>(&vs[(kp * 2) * kVRow + ch * 8]) = v[u][0];
      *reinterpret_cast<u32x4*>(&vs[(kp * 2 + 1) * kVRow + ch * 8]) = v[u][1];
    }
  }
};

// Running softmax state of one wave: 32 query rows.
struct Acc {
  dma::f32x16 o[4];  // O^T: 4 blocks of 32 d x 32 queries
  float m, l;        // base-2 reference and this lane's partial row sum
};

// One gathered chunk of 64 keys for the wave's 32 query rows.  MASKED chunks
// hold keys that only some rows of the tile keep and apply j <= p < e_j per
// element; the others hold keys every row keeps.
template <bool MASKED>
__device__ __forceinline__ void attend_chunk(Acc& acc, const dma::bf16x8 (&qf)[8],
                                             const Smem& sm, int buf, int slot, int lane, int pos,
                                             float scale2) {
  const int l32 = lane & 31, hi = lane >> 5;
  // S^T = K Q^T: rows = the chunk's 64 keys (two blocks of 32), cols = 32 queries
  dma::f32x16 s[2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) s[mb][i] = 0.f;
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const dma::bf16x8 kop = *reinterpret_cast<const dma::bf16x8*>(
          &sm.k[buf][(mb * 32 + l32) * kKRow + kk * 16 + hi * 8]);
      s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qf[kk], s[mb], 0, 0, 0);
    }
  }

  // online softmax over the lane's 32 keys: key(mb, i) = mb*32 + 8*(i/4) + 4*hi + i%4;
  // the other 32 keys of the same query sit in lane ^ 32.
  const float* biasp = &sm.bias[slot][4 * hi];
  const int* pjp = &sm.pj[slot][4 * hi];
  const int* pep = &sm.e[slot][4 * hi];
  float mx = -INFINITY;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int kb = mb * 32 + 8 * q4;
      const float4 bv = *reinterpret_cast<const float4*>(biasp + kb);
      const float bias[4] = {bv.x, bv.y, bv.z, bv.w};
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
        float v = fmaf(s[mb][i], scale2, bias[r]);
        // kept iff pj <= pos < pe, one unsigned compare (pe <= pj: never)
        if constexpr (MASKED)
          v = ((uint32_t)(pos - pj[r]) < (uint32_t)(pe[r] - pj[r])) ? v : -INFINITY;
        s[mb][i] = v;
        mx = fmaxf(mx, v);
      }
    }
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  if (__ballot(mx > acc.m + kLazy) != 0ull) {
    // rare: a logit above the reference by more than the headroom
    const float m_new = fmaxf(acc.m, mx);
    const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(acc.m - m_new);
    acc.l *= alpha;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc.o[db][i] *= alpha;
    acc.m = m_new;
  }
  const float m_use = (acc.m == -INFINITY) ? 0.f : acc.m;
  dma::bf16x8 pb[2][2];  // [mb][half]: B operands of the PV product
  float rs = 0.f;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      float p[8];
#pragma unroll
      for (int t8 = 0; t8 < 8; ++t8) {
        p[t8] = __builtin_amdgcn_exp2f(s[mb][hf * 8 + t8] - m_use);
        rs += p[t8];
      }
      pb[mb][hf] = to_bf16x8(p);
    }
  acc.l += rs;

  // O^T += V^T P^T.  A operand of k-step (mb, hf) for lane (l32, hi): V^T rows
  // d = db*32 + l32, keys mb*32 + 16*hf + 4*hi + [0,4) and mb*32 + 16*hf + 8 +
  // 4*hi + [0,4), matching the keys of P^T's registers.  V stays row-major in
  // LDS; each transposing read serves a 16-lane group g = lane/16: lane r of
  // the group addresses key row kbase + r/4, columns dbase + 16*(g%2) +
  // 4*(r%4), and lane i then receives that group's 4 keys at d = dbase +
  // 16*(g%2) + i.
  const int g = lane >> 4, r = lane & 15;
  // address-space cast of the LDS tile pointer (the instruction takes a local address)
  const __attribute__((address_space(3))) uint16_t* vbase =
      (const __attribute__((address_space(3))) uint16_t*)sm.v[buf];
#pragma unroll
  for (int db = 0; db < 4; ++db) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int k0 = mb * 32 + 16 * hf + 4 * (g >> 1) + (r >> 2);
        const int d0 = db * 32 + 16 * (g & 1) + 4 * (r & 3);
        const i16x4 lo =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vbase + k0 * kVRow + d0));
        const i16x4 up =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vbase + (k0 + 8) * kVRow + d0));
        const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), up2 = __builtin_bit_cast(u32x2, up);
        const u32x4 vv = {lo2[0], lo2[1], up2[0], up2[1]};
        acc.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(dma::bf16x8, vv), pb[mb][hf], acc.o[db], 0, 0, 0);
      }
  }
}

// Workgroup = NH query heads of one kv head x two 32-row halves of a 64-row
// query tile: wave w takes head w/2 and rows (w%2)*32 .. +32.
template <int NH>
__global__ __launch_bounds__(NH * 128, 1) void attn_prefill_bf16_kernel(DmaAttnArgs a) {
  constexpr int NT = NH * 128;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  Smem& sm = *reinterpret_cast<Smem*>(smem_raw);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int G = (int)(a.Hq / a.Hkv);
  const int ngrp = G / NH;
  const int t = blockIdx.x, h = blockIdx.y;
  const int b = blockIdx.z / ngrp, hgrp = blockIdx.z % ngrp;
  const int hq = h * G + hgrp * NH + (wave >> 1);
  const int half = wave & 1;
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
  const uint16_t* Kg = static_cast<const uint16_t*>(a.K) + b * a.ksb + h * a.ksh;
  const uint16_t* Vg = static_cast<const uint16_t*>(a.V) + b * a.ksb + h * a.ksh;
  const float scale2 = a.scale * kLog2e;

  // Q^T operand: lane holds query n = half*32 + l32, d = kk*16 + 8*hi + [0, 8)
  const int n = half * 32 + l32;
  const int pos = p_lo + n;
  dma::bf16x8 qf[8];
  {
    const uint16_t* qrow = static_cast<const uint16_t*>(a.Q) + b * a.qsb + hq * a.qsh +
                           (int64_t)(r_lo + (n < rows ? n : 0)) * a.qss;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      u32x4 v = *reinterpret_cast<const u32x4*>(qrow + kk * 16 + hi * 8);
      if (n >= rows) v = u32x4{0u, 0u, 0u, 0u};
      qf[kk] = __builtin_bit_cast(dma::bf16x8, v);
    }
  }

  Stage<NT> stg;
  // key metadata of the chunk being described (wave 0, one key per lane)
  int jn = -1, en = 0;
  float dn = 0.f;
#define DMA_LOAD_IDX(c_)                   \
  do {                                     \
    const int kk_ = (c_) * kBk + lane;     \
    jn = (kk_ < cnt) ? list[kk_] : -1;     \
  } while (0)
#define DMA_FETCH_META()                   \
  do {                                     \
    const int jj_ = jn < 0 ? 0 : jn;       \
    dn = dl[jj_];                          \
    en = ev[jj_];                          \
  } while (0)
#define DMA_STORE_META(slot_)                                         \
  do {                                                                \
    const bool pad_ = jn < 0;                                         \
    sm.j[slot_][lane] = pad_ ? 0 : jn;                                \
    sm.pj[slot_][lane] = pad_ ? 0x7fffffff : jn;                      \
    sm.e[slot_][lane] = pad_ ? 0 : en;                                \
    sm.bias[slot_][lane] = pad_ ? -INFINITY : (dn - dmax) * kLog2e;   \
  } while (0)

  // prologue: metadata of chunks 0 and 1, K/V of chunk 0, indices of chunk 2
  if (wave == 0 && nch > 0) {
    DMA_LOAD_IDX(0);
    DMA_FETCH_META();
    DMA_STORE_META(0);
    if (nch > 1) {
      DMA_LOAD_IDX(1);
      DMA_FETCH_META();
      DMA_STORE_META(1);
    }
    if (nch > 2) DMA_LOAD_IDX(2);
  }
  __syncthreads();
  if (nch > 0) {
    stg.gather(sm.j[0], Kg, Vg, a.kss, tid);
    stg.store(sm.k[0], sm.v[0], tid);
  }
  __syncthreads();

  Acc acc;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc.o[db][i] = 0.f;
  acc.m = -INFINITY;
  acc.l = 0.f;

  // Chunks [0, nplain) hold only keys every row keeps; the rest need the
  // per-element mask.  Two loops keep the two bodies' registers apart.
#define DMA_CHUNK_LOOP(MASKED, c_from, c_to)                                          \
  for (int c = (c_from); c < (c_to); ++c) {                                           \
    const int buf = c & 1;                                                            \
    /* gather chunk c+1 (indices in slot (c+1)%3) while chunk c is computed;          \
       fetch delta and eviction rows of chunk c+2 (indices loaded last step) */       \
    if (c + 1 < nch) stg.gather(sm.j[(c + 1) % 3], Kg, Vg, a.kss, tid);              \
    if (wave == 0 && c + 2 < nch) DMA_FETCH_META();                                   \
    attend_chunk<MASKED>(acc, qf, sm, buf, c % 3, lane, pos, scale2);                 \
    /* publish chunk c+1; metadata of chunk c+2 goes to slot (c+2)%3, whose chunk     \
       c-1 was last read before the previous barrier */                               \
    if (c + 1 < nch) stg.store(sm.k[buf ^ 1], sm.v[buf ^ 1], tid);                   \
    if (wave == 0 && c + 2 < nch) {                                                   \
      DMA_STORE_META((c + 2) % 3);                                                    \
      if (c + 3 < nch) DMA_LOAD_IDX(c + 3);                                           \
    }                                                                                 \
    __syncthreads();                                                                  \
  }
  DMA_CHUNK_LOOP(false, 0, nplain)
  DMA_CHUNK_LOOP(true, nplain, nch)
#undef DMA_CHUNK_LOOP
#undef DMA_LOAD_IDX
#undef DMA_FETCH_META
#undef DMA_STORE_META

  // epilogue: normalise and write O (and the log-sum-exp)
  const float lt = acc.l + __shfl_xor(acc.l, 32);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (n < rows) {
    uint16_t* orow = static_cast<uint16_t*>(a.O) + (((int64_t)b * a.Sq + r_lo + n) * a.Hq + hq) * kD;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = db * 32 + 8 * q4 + 4 * hi;
        u32x2 u;
        u[0] = pack_bf16x2(acc.o[db][q4 * 4 + 0] * inv, acc.o[db][q4 * 4 + 1] * inv);
        u[1] = pack_bf16x2(acc.o[db][q4 * 4 + 2] * inv, acc.o[db][q4 * 4 + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + d) = u;
      }
    if (a.lse && hi == 0)
      a.lse[((int64_t)b * a.Hq + hq) * a.Sq + r_lo + n] = (acc.m + __log2f(lt)) * kLn2 + dmax;
  }
}

template <int NH>
hipError_t launch(const DmaAttnArgs& a, hipStream_t st) {
  const int G = (int)(a.Hq / a.Hkv);
  dim3 grid((unsigned)a.n_tiles, (unsigned)a.Hkv, (unsigned)(a.B * (G / NH)));
  const size_t lds = sizeof(Smem);
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_prefill_bf16_kernel<NH>),
                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  hipLaunchKernelGGL(attn_prefill_bf16_kernel<NH>, grid, dim3(NH * 128), lds, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t dma_launch_attn_prefill_bf16(const DmaAttnArgs& a, hipStream_t st) {
  const int G = (int)(a.Hq / a.Hkv);
  if (G % 4 == 0) return launch<4>(a, st);
  if (G % 2 == 0) return launch<2>(a, st);
  return launch<1>(a, st);
}
