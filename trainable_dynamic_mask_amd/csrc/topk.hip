// Causal top-w keep mask of the DMA forward (Hugging Face blog "Trainable
// Dynamic Mask Sparse Attention", section "Mask Combination with Causal
// Constraints", m_t = f(top_w(delta + m_c^t))): query position p keeps the w
// keys j <= p with the largest delta, equal delta going to the lower index.
//
// Because delta carries no query index, the keep sets nest: keep(p) is a
// subset of keep(p-1) plus {p}.  So key j is kept on exactly one run of
// positions [j, e_j), where e_j = max(j, b_j) and b_j is the w-th smallest
// index among the keys that beat j (Sk when fewer than w beat it).  The mask
// is built from that form in four steps per (batch, kv head) sequence:
//   T1  sort the keys by the 64-bit composite (delta order, reversed index):
//       bitonic sort of chunks (registers, DPP lane exchanges and LDS), then
//       merge-path merges;
//   T1b rank[j] = position of key j in that order; up to sixteen 1024-key
//       chunks skip the merges: a key's rank is the sum over the chunks of
//       the keys that beat it, found by binary searches over the chunks held
//       in LDS;
//   T2  eviction rows: ranks are cut into blocks of 64; a block builds the
//       bitmap of the indices of all better-ranked keys (a checkpoint bitmap
//       kept every 256 or more ranks plus the keys in between), selects its w-th
//       smallest set bit b, then walks its own ranks in order with one wave:
//       each key gets e = max(j, b) and, when j < b, b steps down to the
//       previous set bit;
//   T3  per 64-row query tile: the union of the rows' keep sets (keys with
//       e_j > max(j, tile start) and j <= tile end), the keys every row keeps
//       first, the natural key tiles touched, and the largest delta; built
//       from candidate lists shared by groups of 8 tiles.
// A single query row (decode) skips T1-T3: one workgroup per sequence finds
// the w-th largest delta by a bitwise search over the order-preserving
// 32-bit codes and compacts the kept keys in index order.
#include "../../include/dma.h"
#include "common.h"
#include "lds_dma.h"

#include <algorithm>
#include <climits>
#include <mutex>

namespace {

// Chunk sizes of the bitonic sort: small chunks (more workgroups, fewer
// stages each) when the ranks come from binary searches over at most
// kRankRunsMax sorted runs, large chunks when merges follow.
constexpr int kSortChunkSmall = 1024;
constexpr int kSortChunkLarge = 4096;
constexpr int kSortPer = 4;  // keys per thread: element i = thread * kSortPer + register
constexpr int kSortRegBits = 2;  // log2(kSortPer)
static_assert((1 << kSortRegBits) == kSortPer, "register bits");
constexpr int kMergeItems = 8;
constexpr int kListRows = 64;   // query rows per tile (Bq)

// ---------------------------------------------------------------- T1: chunk sort
// Value of lane (lane ^ lm) within the wave, for the lane distances the sort
// uses, without the LDS crossbar: DPP row permutations inside 16-lane rows
// (quad permutes for 1, 2, 3; half-row mirror for 7; row mirror for 15; row
// rotate by 8 for 8; 4 = 7 then 3) and the gfx950 row swaps across 16 and 32
// lanes (31 = 15 then 16, 63 = 31 then 32).
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v, int ctrl) {
  switch (ctrl) {  // the control must be an immediate
    case 0xB1: return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);   // quad [1,0,3,2]
    case 0x4E: return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false);   // quad [2,3,0,1]
    case 0x1B: return __builtin_amdgcn_mov_dpp(v, 0x1B, 0xF, 0xF, false);   // quad [3,2,1,0]
    case 0x128: return __builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, false); // row rotate 8
    case 0x140: return __builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, false); // row mirror
    default: return __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, false);    // half-row mirror
  }
}
__device__ __forceinline__ uint32_t swap16_u32(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return (__lane_id() & 16) ? r[0] : r[1];
}
__device__ __forceinline__ uint32_t swap32_u32(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return (__lane_id() & 32) ? r[0] : r[1];
}
__device__ __forceinline__ uint32_t lane_xor_u32(uint32_t v, int lm) {
  switch (lm) {
    case 1: return dpp_u32(v, 0xB1);
    case 2: return dpp_u32(v, 0x4E);
    case 3: return dpp_u32(v, 0x1B);
    case 4: return dpp_u32(dpp_u32(v, 0x141), 0x1B);
    case 7: return dpp_u32(v, 0x141);
    case 8: return dpp_u32(v, 0x128);
    case 15: return dpp_u32(v, 0x140);
    case 16: return swap16_u32(v);
    case 31: return swap16_u32(dpp_u32(v, 0x140));
    case 32: return swap32_u32(v);
    default: return swap32_u32(swap16_u32(dpp_u32(v, 0x140)));  // 63
  }
}
__device__ __forceinline__ uint64_t lane_xor64(uint64_t v, int lm) {
  const uint32_t lo = lane_xor_u32((uint32_t)v, lm);
  const uint32_t hi = lane_xor_u32((uint32_t)(v >> 32), lm);
  return ((uint64_t)hi << 32) | lo;
}
// Bitonic sort (descending) of a CHUNK-key chunk, in the form whose
// comparators all point one way: phase k (block size 2, 4, ..., CHUNK) first
// pairs i with its mirror i ^ (k-1) in the block, then with i ^ j for
// j = k/4, ..., 1, and the lower index of every pair keeps the larger key.
// Element i lives in register i%4 of thread i/4, so pairs at distance < 4 stay
// inside a thread, pairs that differ in bits 2..7 pair lanes of one wave
// (lane_xor64), and only pairs that differ in bits 8 and up cross waves,
// through LDS (two buffers, one barrier each).  Every element is updated by
// its owner, which takes the larger or the smaller of itself and its partner.
// It also writes, per 64-key block of indices, the largest delta code (0 for
// none) for the tile lists' largest deltas.  SOA: the sorted chunks go out as
// 32-bit codes and the low 16 bits of the reversed indices, rows of cstride
// (a multiple of 8) entries, zero past Sk; otherwise as 64-bit keys.
template <int CHUNK, bool SOA>
__global__ __launch_bounds__(CHUNK / kSortPer) void sort_chunk_kernel(
    const float* __restrict__ delta, int Sk, uint64_t* __restrict__ out,
    uint32_t* __restrict__ codes, uint16_t* __restrict__ revs, int cstride,
    uint32_t* __restrict__ blk_code) {
  constexpr int kBits = __builtin_ctz(CHUNK);
  static_assert((1 << kBits) == CHUNK && kBits > kSortRegBits + 6, "chunk spans waves");
  __shared__ uint64_t s[2][CHUNK];
  const int seg = blockIdx.y;
  const int c0 = blockIdx.x * CHUNK;
  const int lane = threadIdx.x & 63;
  const int base = threadIdx.x * kSortPer;
  const float* d = delta + (int64_t)seg * Sk;
  uint64_t a[kSortPer];
#pragma unroll
  for (int r = 0; r < kSortPer; ++r) {
    const int j = c0 + base + r;
    a[r] = (j < Sk) ? dma::key_of(d[j], (uint32_t)j) : 0ull;  // 0 sorts after every real key
  }
  {
    // 16 lanes (one DPP row) hold a 64-key block
    uint32_t bc = 0u;
#pragma unroll
    for (int r = 0; r < kSortPer; ++r) bc = max(bc, (uint32_t)(a[r] >> 32));
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) bc = max(bc, (uint32_t)__shfl_xor((int)bc, o));
    const int nblk = (Sk + 63) >> 6;
    if ((lane & 15) == 0 && c0 + base < Sk) blk_code[(int64_t)seg * nblk + ((c0 + base) >> 6)] = bc;
  }
  int lds_stage = 0;  // LDS stages alternate buffers, so a buffer is rewritten
                      // only after the barrier of the stage in between
#pragma unroll
  for (int m = 1; m <= kBits; ++m) {
#pragma unroll
    for (int b = m - 1; b >= 0; --b) {
      // partner = i ^ x; the pair's lower index has bit b clear
      const int x = b == m - 1 ? (1 << m) - 1 : 1 << b;
      if (b < kSortRegBits) {
        // both elements belong to this thread
#pragma unroll
        for (int r = 0; r < kSortPer; ++r) {
          if (r & (1 << b)) continue;
          const uint64_t u = a[r], v = a[r ^ x];
          const bool gt = u > v;
          a[r] = gt ? u : v;
          a[r ^ x] = gt ? v : u;
        }
      } else if (b < kSortRegBits + 6) {
        // partner lane = lane ^ (x >> reg bits), partner register = r ^ (x % kSortPer)
        const int lm = x >> kSortRegBits;
        const bool lower = (lane & (1 << (b - kSortRegBits))) == 0;
        uint64_t p[kSortPer];
#pragma unroll
        for (int r = 0; r < kSortPer; ++r) p[r] = lane_xor64(a[r ^ (x & (kSortPer - 1))], lm);
#pragma unroll
        for (int r = 0; r < kSortPer; ++r) a[r] = ((a[r] > p[r]) == lower) ? a[r] : p[r];
      } else {
        uint64_t* sb = s[lds_stage & 1];
        ++lds_stage;
#pragma unroll
        for (int r = 0; r < kSortPer; ++r) sb[base + r] = a[r];
        __syncthreads();
        const bool lower = (base & (1 << b)) == 0;
#pragma unroll
        for (int r = 0; r < kSortPer; ++r) {
          const uint64_t p = sb[(base + r) ^ x];
          a[r] = ((a[r] > p) == lower) ? a[r] : p;
        }
      }
    }
  }
  if (SOA) {
    static_assert(kSortPer == 4, "one 16-byte and one 8-byte store per thread");
    const int q = c0 + base;
    if (q < cstride) {
      *reinterpret_cast<uint4*>(codes + (int64_t)seg * cstride + q) =
          make_uint4((uint32_t)(a[0] >> 32), (uint32_t)(a[1] >> 32), (uint32_t)(a[2] >> 32),
                     (uint32_t)(a[3] >> 32));
      *reinterpret_cast<uint2*>(revs + (int64_t)seg * cstride + q) =
          make_uint2((a[0] & 0xffffu) | ((uint32_t)a[1] << 16),
                     (a[2] & 0xffffu) | ((uint32_t)a[3] << 16));
    }
  } else {
    uint64_t* o = out + (int64_t)seg * Sk;
#pragma unroll
    for (int r = 0; r < kSortPer; ++r)
      if (c0 + base + r < Sk) o[c0 + base + r] = a[r];
  }
}

// ---------------------------------------------------------------- T1: merge
// Merge neighbouring descending runs of length L into runs of 2L.
__global__ __launch_bounds__(256) void merge_kernel(const uint64_t* __restrict__ src,
                                                    uint64_t* __restrict__ dst, int Sk, int L) {
  const int seg = blockIdx.y;
  const int64_t o_glob = ((int64_t)blockIdx.x * 256 + threadIdx.x) * kMergeItems;
  if (o_glob >= Sk) return;
  const int base = (int)(o_glob / (2 * L)) * (2 * L);
  const int o = (int)o_glob - base;
  const int la = min(L, Sk - base);
  const int lb = max(0, min(L, Sk - base - L));
  const uint64_t* A = src + (int64_t)seg * Sk + base;
  const uint64_t* B = A + L;
  // co-rank: number of A elements among the first o outputs
  int lo = max(0, o - lb), hi = min(o, la);
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (A[mid] > B[o - mid - 1]) lo = mid + 1;
    else hi = mid;
  }
  int ia = lo, ib = o - lo;
  uint64_t* D = dst + (int64_t)seg * Sk + base + o;
  const int n = min(kMergeItems, la + lb - o);
  for (int k = 0; k < n; ++k) {
    const bool takeA = (ib >= lb) || (ia < la && A[ia] > B[ib]);
    D[k] = takeA ? A[ia++] : B[ib++];
  }
}

// ---------------------------------------------------------------- T1b: ranks
__global__ __launch_bounds__(256) void rank_kernel(const uint64_t* __restrict__ sorted, int Sk,
                                                   int rstride, int32_t* __restrict__ rank) {
  const int seg = blockIdx.y;
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= Sk) return;
  const uint32_t j = dma::index_of(sorted[(int64_t)seg * Sk + r]);
  rank[(int64_t)seg * rstride + j] = r;
}

// T1 + T1b for a sequence of at most kRankRunsMax sorted runs of
// kSortChunkSmall keys, in place of the merges: the rank of a key is the
// number of keys that beat it, summed over the runs (its own run included,
// where the count is its position; keys are distinct, so each count is a
// binary search).  A workgroup holds every run of its sequence in LDS and
// ranks kRankRunsKeys consecutive keys of one run (similar keys, so the
// searches of a wave read nearby LDS words); it writes rank[j] and the merged
// order.  The searches compare the 32-bit delta codes only (runs padded to
// full length with code 0, which beats nothing); where a search stops on a
// key of equal code, the keys of equal code are resolved by a second search
// on the low 16 bits of the reversed index (Sk <= 16384, so those order the
// indices).
constexpr int kRankRunsMax = 16;
constexpr int kRankRunsThreads = 256;
constexpr int kRankRunsU = 2;  // keys per thread
constexpr int kRankRunsKeys = kRankRunsThreads * kRankRunsU;
static_assert(kSortChunkSmall % kRankRunsKeys == 0, "a workgroup's keys lie in one run");
static_assert(kRankRunsMax * kSortChunkSmall <= 65536, "16-bit reversed indices");

template <int NR>  // runs searched (>= the sequence's run count)
__global__ __launch_bounds__(kRankRunsThreads) void rank_runs_kernel(
    const uint32_t* __restrict__ codes, const uint16_t* __restrict__ revs, int cstride, int Sk,
    int rstride, int32_t* __restrict__ rank, uint64_t* __restrict__ merged, int nseg) {
  constexpr int kRun = kSortChunkSmall;
  constexpr int kN = NR * kRun;
  extern __shared__ __align__(16) uint32_t s_code[];            // [kN] delta codes
  uint16_t* s_rev = reinterpret_cast<uint16_t*>(s_code + kN);  // [kN] reversed index, low 16 bits
  // workgroup i runs on XCD i % 8: with the sequence as the fast index, the
  // workgroups of a sequence share one XCD's L2, which then holds its runs
  const int id = blockIdx.x;
  const int seg = id % nseg, bx = id / nseg;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int kWaves = kRankRunsThreads / 64;
  {
    // the runs into LDS by direct 16-byte loads (1 KB per wave and load):
    // codes, then reversed indices; loads past the row read its start, and
    // those LDS words are cleared once the loads have landed
    const uint32_t* cg = codes + (int64_t)seg * cstride;
    const uint16_t* rg = revs + (int64_t)seg * cstride;
    constexpr int kCodeLoads = kN * 4 / 1024 / kWaves, kRevLoads = kN * 2 / 1024 / kWaves;
    const int uw = __builtin_amdgcn_readfirstlane(wave);  // m0 takes a scalar address
#pragma unroll
    for (int t = 0; t < kCodeLoads; ++t) {
      const int blk = uw + kWaves * t;  // 256 codes each
      const int g = 256 * blk + 4 * lane;
      dma::dma_b128(cg + (g + 4 <= cstride ? g : 0), dma::lds_addr(s_code + 256 * blk));
    }
#pragma unroll
    for (int t = 0; t < kRevLoads; ++t) {
      const int blk = uw + kWaves * t;  // 512 reversed indices each
      const int g = 512 * blk + 8 * lane;
      dma::dma_b128(rg + (g + 8 <= cstride ? g : 0), dma::lds_addr(s_rev + 512 * blk));
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    for (int i = cstride + tid; i < kN; i += kRankRunsThreads) {
      s_code[i] = 0u;
      s_rev[i] = 0;
    }
    __syncthreads();
  }

  const int r = bx / (kRun / kRankRunsKeys);
  const int q0 = r * kRun + (bx % (kRun / kRankRunsKeys)) * kRankRunsKeys + tid;
  uint32_t c[kRankRunsU];
  uint16_t rv[kRankRunsU];
  uint32_t off[kRankRunsU][NR];  // LDS byte offset: run base plus 4 x the count so far
#pragma unroll
  for (int u = 0; u < kRankRunsU; ++u) {
    const int q = min(q0 + u * kRankRunsThreads, Sk - 1);
    c[u] = s_code[q];
    rv[u] = s_rev[q];
#pragma unroll
    for (int o = 0; o < NR; ++o) off[u][o] = 4u * (uint32_t)(o * kRun);
  }
  const char* sc = reinterpret_cast<const char*>(s_code);
  // all kRankRunsU x NR searches of a thread advance together, one halving
  // step at a time; the first kRun - 1 keys of a run, then the last one
#pragma unroll
  for (int step = kRun / 2; step > 0; step >>= 1) {
#pragma unroll
    for (int o = 0; o < NR; ++o) {
      uint32_t v[kRankRunsU];
#pragma unroll
      for (int u = 0; u < kRankRunsU; ++u)
        v[u] = *reinterpret_cast<const uint32_t*>(sc + off[u][o] + 4 * (step - 1));
#pragma unroll
      for (int u = 0; u < kRankRunsU; ++u) off[u][o] |= v[u] > c[u] ? 4u * step : 0u;
    }
  }
  uint32_t tie[kRankRunsU];  // bit o: the search stopped on a key of equal code
#pragma unroll
  for (int u = 0; u < kRankRunsU; ++u) {
    tie[u] = 0u;
#pragma unroll
    for (int o = 0; o < NR; ++o) {
      const uint32_t v = *reinterpret_cast<const uint32_t*>(sc + off[u][o]);
      off[u][o] += v > c[u] ? 4u : 0u;
      tie[u] |= (v == c[u] ? 1u : 0u) << o;
    }
  }
#pragma unroll
  for (int u = 0; u < kRankRunsU; ++u) {
    int pos = 0;
#pragma unroll
    for (int o = 0; o < NR; ++o) pos += (int)(off[u][o] >> 2) - o * kRun;
    // equal codes: the keys of run o from the count on with that code and a
    // lower index (larger reversed index) also beat the key
    for (uint32_t t = tie[u]; t; t &= t - 1u) {
      const int o = __builtin_ctz(t);
      const int n_o = min(kRun, Sk - o * kRun);
      const int c0 = (int)(off[u][o] >> 2);
      int lo = c0, hi = o * kRun + n_o;  // first position that does not beat
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (s_code[mid] == c[u] && s_rev[mid] > rv[u]) lo = mid + 1;
        else hi = mid;
      }
      pos += lo - c0;
    }
    const int q = q0 + u * kRankRunsThreads;
    if (q < Sk) {
      // the key itself, rebuilt from its code and index (which fits 16 bits)
      const uint32_t j = 0xffffu - (uint32_t)rv[u];
      rank[(int64_t)seg * rstride + j] = pos;
      merged[(int64_t)seg * Sk + pos] = ((uint64_t)c[u] << 32) | (uint64_t)(0xffffffffu - j);
    }
  }
}

// Exclusive prefix sum over a block of NT threads (NT/64 waves); also returns the total.
template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int* s_w, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) s_w[wave] = x;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int k = 0; k < NT / 64; ++k) {
    const int t = s_w[k];
    if (k < wave) before += t;
    total += t;
  }
  __syncthreads();
  return before + x - v;
}

// ---------------------------------------------------------------- T2: eviction rows
// T2a: checkpoint bitmaps { j : rank[j] < c * chk } for c = 1 .. n_chk-1
// (at most 64), nwr words each, so an eviction block needs at most chk-1
// insertions on top of one.  One wave per 64 consecutive indices: a ballot
// per checkpoint, and lane c-1 stores the two words of checkpoint c.
__global__ __launch_bounds__(256) void ckpt_kernel(const int32_t* __restrict__ rank, int Sk,
                                                   int rstride, int chk, int n_chk, int nwr,
                                                   uint32_t* __restrict__ ckpt) {
  const int seg = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int j0 = blockIdx.x * 256 + (int)threadIdx.x - lane;  // the wave's first index
  if (j0 >= nwr * 32) return;  // past the padded words (wave-uniform)
  const int j = j0 + lane;
  const int r = j < Sk ? rank[(int64_t)seg * rstride + j] : INT_MAX;
  uint64_t mine = 0ull;
  for (int c = 1; c < n_chk; ++c) {
    const uint64_t b = dma::ballot(r < c * chk);
    mine = lane == c - 1 ? b : mine;
  }
  // nwr is a multiple of 4 and j0 of 64: the two words are 8-byte aligned
  if (lane < n_chk - 1)
    *reinterpret_cast<uint64_t*>(ckpt + ((int64_t)seg * n_chk + lane + 1) * nwr + (j0 >> 5)) =
        mine;
}

// T2b: eviction rows, one block of 64 consecutive ranks per wave.
//
// The block's keys are taken in rank order, k = 0..63, key k with index x_k.
// Let f_k be the w-th smallest index among the keys of rank < rs + k (the
// bitmap S plus x_0..x_{k-1}); then e_k = max(x_k, f_k), and f moves only
// when a key with x_k < f_k (a mover) arrives: to the largest index below
// f_k in S plus the movers so far (x_k itself qualifies).  Let M be the 64
// largest indices of S at or below f_0, descending (M[0] = f_0).  After t
// moves, f is entry t of M with the movers inserted in order (a mover enters
// below the current f, so entries 0..t are final once t moves are made).  A
// key with x < M[63] is a mover whatever happened before it, and enters
// below every entry f reaches in 64 keys, so it only counts as a move; keys
// with M[63] <= x < f_0 are decided one at a time in rank order against
// M[t], and the movers among them are inserted into M (a lane-parallel
// shift).  Then mover k gets e_k = M[t_k], with t_k the movers before it.
//
// m: M, one entry per lane (-1 past the w-th set bit); xl: the block's key
// indices, INT_MAX past the block.  Returns e for this lane's key.
__device__ __forceinline__ int evict_walk(int m, int xl) {
  const int lane = dma::lane_id();
  const int f0 = __builtin_amdgcn_readfirstlane(__shfl(m, 0));
  const int m63 = __shfl(m, 63);                             // -1 when w < 64
  const uint64_t sure = dma::ballot(xl < m63);               // movers whatever came before
  const uint64_t open = dma::ballot(xl >= m63 && xl < f0);   // decided in order
  uint64_t movers = sure;
  for (uint64_t o = open; o; o &= o - 1ull) {
    const int u = __builtin_ctzll(o);
    const int t = __popcll(movers & ((1ull << u) - 1ull));  // moves before key u
    const int f = __shfl(m, t);
    const int xu = __shfl(xl, u);
    if (xu < f) {  // wave-uniform
      movers |= 1ull << u;
      // insert xu below entry t: entries below xu move down one lane
      const int up = __shfl_up(m, 1);
      m = m > xu ? m : ((lane == 0 || up > xu) ? xu : up);
    }
  }
  const bool mv = (movers >> lane) & 1ull;
  const int fk = __shfl(m, dma::rank_below(movers));  // f when key k arrives
  return mv ? fk : xl;
}

// Orders one wave's LDS accesses across its lanes (no instruction: the
// compiler keeps them in program order; the wave executes LDS in order).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
}

// M from one wave's bitmap of nw words in LDS (at least w set bits): lane i
// gets the set bit of ascending position w-1-i (0-based), -1 where there is
// none (w < 64).  Per-word exclusive prefix counts go to s_pre (nw ints of
// LDS); each lane then finds its word by a binary search over them (the last
// word whose prefix is at most its position) and its bit by halving selects.
__device__ __forceinline__ int wave_top_m(const uint32_t* bm, int nw, int w, int* s_pre) {
  const int lane = dma::lane_id();
  const int per = (nw + 63) >> 6;
  const int wlo = min(nw, lane * per), whi = min(nw, wlo + per);
  int cnt = 0;
  for (int k = wlo; k < whi; ++k) cnt += __popc(bm[k]);
  int incl = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  int run = incl - cnt;
  for (int k = wlo; k < whi; ++k) {
    s_pre[k] = run;
    run += __popc(bm[k]);
  }
  wave_lds_sync();
  const int P = w - 1 - lane;
  if (P < 0) return -1;
  int lo = 0, hi = nw - 1;  // s_pre[lo] <= P
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_pre[mid] <= P) lo = mid;
    else hi = mid - 1;
  }
  uint32_t x = bm[lo];
  int r = P - s_pre[lo];  // r-th set bit of word lo (0-based)
  int b = 0;
#pragma unroll
  for (int h = 16; h >= 1; h >>= 1) {
    const int c = __popc(x & ((1u << h) - 1u));
    if (r >= c) {
      r -= c;
      x >>= h;
      b += h;
    }
  }
  return lo * 32 + b;
}

// Eviction rows of the ranks [R0, R0 + 256), four blocks of 64, one per
// wave.  The workgroup builds the bitmap of the ranks below R0 once (the
// checkpoint below R0 plus the ranks in between; none when the checkpoints
// are 256 ranks apart), then each wave copies it, adds the workgroup's ranks
// below its own block, and walks its block with no further barrier.
constexpr int kEvictWG = 4;  // blocks (waves) per workgroup
constexpr int kEvictRanks = 64 * kEvictWG;

__global__ __launch_bounds__(kEvictRanks) void evict_wg_kernel(
    const uint64_t* __restrict__ sorted, int Sk, int w, int chk, int n_chk, int nwr,
    const uint32_t* __restrict__ ckpt, int32_t* __restrict__ evict) {
  extern __shared__ __align__(16) uint32_t s_lds[];
  uint32_t* s_base = s_lds;                                    // [nwr] ranks < R0
  uint32_t* s_bm = s_lds + nwr;                                // [kEvictWG][nwr] bitmaps
  int* s_pre = reinterpret_cast<int*>(s_bm + kEvictWG * nwr);  // [kEvictWG][nwr] prefixes
  int* s_x = s_pre + kEvictWG * nwr;                           // [kEvictRanks] indices
  const int seg = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t* K = sorted + (int64_t)seg * Sk;
  int32_t* E = evict + (int64_t)seg * Sk;
  const int R0 = blockIdx.x * kEvictRanks;
  const int r = R0 + tid;  // this thread's rank
  const int x = r < Sk ? (int)dma::index_of(K[r]) : INT_MAX;
  const int c = R0 / chk;
  const uint32_t* cp = ckpt + ((int64_t)seg * n_chk + c) * nwr;
  for (int k = tid; k < nwr; k += kEvictRanks) s_base[k] = c > 0 ? cp[k] : 0u;
  s_x[tid] = x;
  if (r < min(Sk, w)) E[x] = Sk;  // the w best keys are kept to the end
  __syncthreads();
  if (c * chk < R0) {  // block-uniform
    for (int q = c * chk + tid; q < R0; q += kEvictRanks) {
      const uint32_t xi = dma::index_of(K[q]);
      atomicOr(&s_base[xi >> 5], 1u << (xi & 31));
    }
    __syncthreads();
  }
  // ---- per wave: its block of ranks [b0, b1), walked from rs
  const int b0 = R0 + 64 * wave, b1 = min(Sk, b0 + 64);
  const int rsw = max(b0, w);
  if (rsw >= b1) return;  // wave-uniform; no block barrier follows
  uint32_t* bm = s_bm + wave * nwr;
  for (int k = lane; k < nwr; k += 64) bm[k] = s_base[k];
  wave_lds_sync();
  for (int q = lane; q < rsw - R0; q += 64) {  // ranks R0 .. rsw-1
    const int xi = s_x[q];
    atomicOr(&bm[xi >> 5], 1u << (xi & 31));
  }
  wave_lds_sync();
  const int m = wave_top_m(bm, (Sk + 31) >> 5, w, s_pre + wave * nwr);
  const int xl = rsw + lane < b1 ? s_x[rsw - R0 + lane] : INT_MAX;
  const int e = evict_walk(m, xl);
  if (rsw + lane < b1) E[xl] = e;
}

// Eviction rows of the keys of ranks [r0, r0 + 64), one block per
// workgroup, for large Sk (the per-wave bitmap copies of evict_wg_kernel
// would not fit LDS).  Every global load of the block (its keys, the
// checkpoint words, the keys of the ranks between the checkpoint and the
// block) is issued before the first is used.
constexpr int kEvictR = 64;  // ranks per block: one wave's keys
constexpr int kEvictThreads = 256;
constexpr int kEvictWordsPer = 8;  // checkpoint words per thread and load batch
constexpr int kEvictInsPer = 4;    // inserted keys per thread and load batch

__global__ __launch_bounds__(kEvictThreads) void evict_kernel(
    const uint64_t* __restrict__ sorted, int Sk, int w, int chk, int n_chk, int nwr,
    const uint32_t* __restrict__ ckpt, int32_t* __restrict__ evict) {
  // Dynamic LDS only: bitmap of indices (nwr words), s_w[8] (scan slots),
  // s_m[64] (M).
  extern __shared__ __align__(16) uint32_t bm[];
  int* s_w = reinterpret_cast<int*>(bm + nwr);
  int* s_m = s_w + 8;
  const int seg = blockIdx.y;
  const int tid = threadIdx.x;
  const uint64_t* K = sorted + (int64_t)seg * Sk;
  int32_t* E = evict + (int64_t)seg * Sk;
  const int lane = tid & 63, wave = tid >> 6;
  const int r0 = blockIdx.x * kEvictR, r1 = min(Sk, r0 + kEvictR);
  // the w best keys are never beaten by w others: kept to the end
  for (int r = r0 + tid; r < min(r1, w); r += kEvictThreads) E[dma::index_of(K[r])] = Sk;
  const int rs = max(r0, w);
  if (rs >= r1) return;

  // Bitmap of { j : rank[j] < rs }: the nearest checkpoint below rs, then
  // the keys of the ranks in between.
  const int c = rs / chk;
  const int ri0 = c * chk;  // first rank inserted on top of the checkpoint
  const uint32_t* cp = ckpt + ((int64_t)seg * n_chk + c) * nwr;
  const uint64_t kw = (wave == 0 && rs + lane < r1) ? K[rs + lane] : 0ull;
  uint64_t iv[kEvictInsPer];
#pragma unroll
  for (int u = 0; u < kEvictInsPer; ++u) {
    const int r = ri0 + u * kEvictThreads + tid;
    iv[u] = r < rs ? K[r] : 0ull;
  }
  if (tid < 64) s_m[tid] = -1;  // entries past the w-th (w < 64)
  for (int k0 = 0; k0 < nwr; k0 += kEvictThreads * kEvictWordsPer) {
    uint32_t wv[kEvictWordsPer];
#pragma unroll
    for (int u = 0; u < kEvictWordsPer; ++u) {
      const int k = k0 + u * kEvictThreads + tid;
      wv[u] = (c > 0 && k < nwr) ? cp[k] : 0u;
    }
#pragma unroll
    for (int u = 0; u < kEvictWordsPer; ++u) {
      const int k = k0 + u * kEvictThreads + tid;
      if (k < nwr) bm[k] = wv[u];
    }
  }
  __syncthreads();  // every word is written before the first insertion
  for (int i0 = ri0; i0 < rs; i0 += kEvictThreads * kEvictInsPer) {
    if (i0 != ri0) {
#pragma unroll
      for (int u = 0; u < kEvictInsPer; ++u) {
        const int r = i0 + u * kEvictThreads + tid;
        iv[u] = r < rs ? K[r] : 0ull;
      }
    }
#pragma unroll
    for (int u = 0; u < kEvictInsPer; ++u) {
      const int r = i0 + u * kEvictThreads + tid;
      if (r < rs) {
        const uint32_t x = dma::index_of(iv[u]);
        atomicOr(&bm[x >> 5], 1u << (x & 31));
      }
    }
  }
  __syncthreads();

  // M: set bits of ascending positions w-64 .. w-1 (0-based), from
  // per-thread popcounts and one block scan; M[i] is position w-1-i.
  const int nw = (Sk + 31) >> 5;
  const int per = (nw + kEvictThreads - 1) / kEvictThreads;
  const int wlo = min(nw, tid * per), whi = min(nw, wlo + per);
  int cnt = 0;
  for (int k = wlo; k < whi; ++k) cnt += __popc(bm[k]);
  int total;
  const int before = block_excl_scan<kEvictThreads>(cnt, s_w, total);
  const int plo = max(0, w - 64);
  if (before < w && before + cnt > plo) {
    int p = before;
    for (int k = wlo; k < whi && p < w; ++k) {
      uint32_t x = bm[k];
      const int cc = __popc(x);
      if (p + cc <= plo) {
        p += cc;
        continue;
      }
      for (; x && p < w; x &= x - 1u, ++p)
        if (p >= plo) s_m[w - 1 - p] = k * 32 + __builtin_ctz(x);
    }
  }
  __syncthreads();
  if (wave != 0) return;
  // total >= rs >= w set bits, so M[0] = f_0 is a real index
  const int steps = r1 - rs;  // 1..64 keys
  const int xl = lane < steps ? (int)dma::index_of(kw) : INT_MAX;
  const int e = evict_walk(s_m[lane], xl);
  if (lane < steps) E[xl] = e;
}

// ---------------------------------------------------------------- T3: tile lists
// Two levels.  Membership in a tile's union is a run of consecutive tiles
// starting at the key's own tile (j is in U_t iff j <= p_hi(t) and
// e_j > max(j, p_lo(t)), and p_lo grows with t), so the keys in the union of
// any tile of a group of kSuperTiles (8) consecutive tiles are
//   C = { j <= P_hi : e_j > max(j, P_lo) }
// with P_lo, P_hi the group's first and last position: the min(w, P_lo+1)
// keys kept at P_lo plus the keys born inside the group with e_j > j, at most
// w + 511.  L1 builds C once per group by scanning keys 0..P_hi; L2 builds
// the group's tile lists from C only, instead of rescanning each tile's whole
// prefix.  Both keep ascending key order.
constexpr int kListWaves = 16;  // L1: 16 waves x 16 x 64 keys per load batch
constexpr int kListUnroll = 16;
constexpr int kSuperTiles = 8;

// L1.  Wave w scans keys [w*L, (w+1)*L) of 0..P_hi, 16 x 64 keys per step
// with all loads issued first (one step covers 16K keys per workgroup).
// Pass 1 counts, one barrier turns counts into offsets, pass 2 writes the
// members' index and eviction row.  Pass 2 also gives each tile of the group
// its largest delta, the largest over keys 0..p_hi (that key is kept by row
// p_hi, so it is also the largest over U).
__global__ __launch_bounds__(kListWaves * 64) void cand_kernel(
    const float* __restrict__ delta, const int32_t* __restrict__ evict, int Sk, int Sq, int q0,
    int n_super, int n_tiles, int cap, int32_t* __restrict__ cj, int32_t* __restrict__ ce,
    int32_t* __restrict__ ccnt, float* __restrict__ u_dmax, float* __restrict__ u_dlo) {
  __shared__ int s_c[kListWaves];
  // order codes of the largest delta per bucket: bucket i holds the keys of
  // tile t0+i's own rows, bucket kSuperTiles every key before the group
  __shared__ uint32_t s_b[kSuperTiles + 1];
  if (threadIdx.x <= kSuperTiles) s_b[threadIdx.x] = 0u;  // 0: below every code
  const int seg = blockIdx.y, T = blockIdx.x;
  const int64_t g = (int64_t)seg * n_super + T;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int P_lo = q0 + T * kSuperTiles * kListRows;
  const int P_hi = q0 + min(Sq, (T + 1) * kSuperTiles * kListRows) - 1;
  const int32_t* E = evict + (int64_t)seg * Sk;
  const float* Dl = delta + (int64_t)seg * Sk;
  const int n = P_hi + 1;
  const int L = ((n + 64 * kListWaves - 1) / (64 * kListWaves)) * 64;
  const int j0 = min(n, wave * L), j1 = min(n, j0 + L);

  int nc = 0;
  for (int jb = j0; jb < j1; jb += 64 * kListUnroll) {
    int e[kListUnroll];
#pragma unroll
    for (int u = 0; u < kListUnroll; ++u) {
      const int j = jb + u * 64 + lane;
      e[u] = j < j1 ? E[j] : 0;
    }
#pragma unroll
    for (int u = 0; u < kListUnroll; ++u) {
      const int j = jb + u * 64 + lane;
      nc += __popcll(dma::ballot(j < j1 && e[u] > max(j, P_lo)));
    }
  }
  if (lane == 0) s_c[wave] = nc;
  __syncthreads();
  int oc = 0, tc = 0;
#pragma unroll
  for (int k = 0; k < kListWaves; ++k) {
    if (k < wave) oc += s_c[k];
    tc += s_c[k];
  }
  int32_t* oj = cj + g * cap;
  int32_t* oe = ce + g * cap;
  uint32_t m0 = 0u;  // this lane's largest code before the group
  for (int jb = j0; jb < j1; jb += 64 * kListUnroll) {
    int e[kListUnroll];
    float d[kListUnroll];
#pragma unroll
    for (int u = 0; u < kListUnroll; ++u) {
      const int j = jb + u * 64 + lane;
      e[u] = j < j1 ? E[j] : 0;
      d[u] = j < j1 ? Dl[j] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kListUnroll; ++u) {
      const int j = jb + u * 64 + lane;
      const bool member = j < j1 && e[u] > max(j, P_lo);
      const uint64_t bm = dma::ballot(member);
      if (member) {
        const int pos = oc + dma::rank_below(bm);
        if (pos < cap) {
          oj[pos] = j;
          oe[pos] = e[u];
        }
      }
      if (j < j1) {
        if (j < P_lo)
          m0 = max(m0, dma::ord32(d[u]));
        else
          atomicMax(&s_b[(j - P_lo) >> 6], dma::ord32(d[u]));
      }
      oc += __popcll(bm);
    }
  }
  if (threadIdx.x == 0) ccnt[g] = min(tc, cap);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m0 = max(m0, (uint32_t)__shfl_xor((int)m0, o));
  if (lane == 0) atomicMax(&s_b[kSuperTiles], m0);
  __syncthreads();
  // tile t0+i: the largest delta over keys 0..p_hi (the keys before the
  // group and buckets 0..i), and over the keys before its first row (before
  // the group and buckets 0..i-1; minus infinity when there are none: code 0)
  const int t0 = T * kSuperTiles;
  const int i = threadIdx.x;
  if (i < min(kSuperTiles, n_tiles - t0)) {
    uint32_t mlo = s_b[kSuperTiles];
    for (int k = 0; k < i; ++k) mlo = max(mlo, s_b[k]);
    const uint32_t m = max(mlo, s_b[i]);
    auto value = [](uint32_t c) {  // inverse of ord32
      return c == 0u ? -INFINITY
                     : __uint_as_float((c & 0x80000000u) ? (c & 0x7fffffffu) : ~c);
    };
    u_dmax[(int64_t)seg * n_tiles + t0 + i] = value(m);
    if (u_dlo) u_dlo[(int64_t)seg * n_tiles + t0 + i] = value(mlo);
  }
}

// L2.  One workgroup per group writes the lists of all its tiles: each
// candidate is tested against every tile of the group at once (its member
// tiles and the tiles whose every row keeps it), and per-tile ballots give
// exact positions in both ascending runs.  Pass 1 counts per tile and wave
// and marks the key tiles in LDS bitmaps; one barrier turns the counts into
// offsets; pass 2 writes.
constexpr int kGroupWaves = 8;
constexpr int kGroupUnroll = 8;  // staged per wave: 8 x 64 candidates (8 waves: 4096)
constexpr int kMaxKtWords = DMA_MAX_SK / DMA_BLOCK_K / 32;

__global__ __launch_bounds__(kGroupWaves * 64) void group_lists_kernel(
    const int32_t* __restrict__ cj, const int32_t* __restrict__ ce,
    const int32_t* __restrict__ ccnt, int Sq, int q0, int n_tiles, int n_super, int cap,
    int u_stride, int kt_stride, int32_t* __restrict__ u_idx, int32_t* __restrict__ u_cnt,
    int32_t* __restrict__ u_nfull, int32_t* __restrict__ kt_idx, int32_t* __restrict__ kt_cnt) {
  extern __shared__ uint32_t s_kt[];  // per tile of the group: key-tile bitmap of kw words
  __shared__ int s_c[kGroupWaves][kSuperTiles][2];
  __shared__ int s_sj[kGroupWaves][64 * kGroupUnroll];
  __shared__ int s_se[kGroupWaves][64 * kGroupUnroll];
  const int seg = blockIdx.y, T = blockIdx.x;
  const int64_t gs = (int64_t)seg * n_super + T;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = T * kSuperTiles;
  const int ng = min(kSuperTiles, n_tiles - t0);  // tiles in this group
  const int P_lo = q0 + t0 * kListRows;
  const int Pend = q0 + Sq - 1;  // last position
  const int nc = ccnt[gs];
  const int32_t* Cj = cj + gs * cap;
  const int32_t* Ce = ce + gs * cap;
  const int kw = kt_idx ? (kt_stride + 31) / 32 : 0;
  for (int k = threadIdx.x; k < ng * kw; k += kGroupWaves * 64) s_kt[k] = 0u;
  const int L = ((nc + 64 * kGroupWaves - 1) / (64 * kGroupWaves)) * 64;
  const int k0 = min(nc, wave * L), k1 = min(nc, k0 + L);
  __syncthreads();

  // Member and full tile masks of one candidate (bit i: tile t0 + i), in
  // closed form: with r = j - P_lo, key j is in U of tile i iff e > j,
  // j <= Pend and floor(r/64) <= i <= floor((e-1-P_lo)/64); every row of
  // tile i keeps it iff also ceil(r/64) <= i and (e > Pend or
  // i <= floor((e-64-P_lo)/64)).
  auto span = [](int a, int b) -> uint32_t {  // bits a..b
    return (a > b || b < 0) ? 0u : (uint32_t)((2ull << b) - (1ull << a));
  };
  auto masks = [&](int j, int e, bool valid, uint32_t& mm, uint32_t& mf) {
    const int r = j - P_lo;
    const bool any = valid && e > j && j <= Pend;
    mm = any ? span(r < 0 ? 0 : r >> 6, min((e - 1 - P_lo) >> 6, ng - 1)) : 0u;
    const int fb = e > Pend ? ng - 1 : min((e - 64 - P_lo) >> 6, ng - 1);
    mf = mm & span(r <= 0 ? 0 : (r + 63) >> 6, fb);
  };

  // Each wave stages up to 64*kGroupUnroll of its candidates at a time in a
  // private LDS region, with all global loads issued together, then walks
  // them 64 at a time.
  auto stage = [&](int kb) {
    int jv[kGroupUnroll], ev[kGroupUnroll];
#pragma unroll
    for (int u = 0; u < kGroupUnroll; ++u) {  // clamped positions, validity applied later
      const int k = min(kb + u * 64 + lane, k1 - 1);
      jv[u] = Cj[k];
      ev[u] = Ce[k];
    }
#pragma unroll
    for (int u = 0; u < kGroupUnroll; ++u) {
      s_sj[wave][u * 64 + lane] = jv[u];
      s_se[wave][u * 64 + lane] = ev[u];
    }
  };

  // Key tiles touched by tile i's members: runs of lanes with one key tile
  // (candidates ascend), marked by the run's first lane when any lane of the
  // run is a member.
  auto run_mask = [&](int j, uint64_t& runm) -> bool {
    const int kt = j >> 6;
    const int ktp = __shfl_up(kt, 1);
    const bool start = lane == 0 || ktp != kt;
    const uint64_t rs = dma::ballot(start);
    const uint64_t above = lane == 63 ? 0ull : rs & (~0ull << (lane + 1));
    const uint64_t upto = above ? (above & (0ull - above)) - 1ull : ~0ull;  // bits below next start
    runm = upto & (~0ull << lane);
    return start;
  };

  // per-tile counts and offsets live in lane i of the wave (tile t0 + i)
  int nfv = 0, npv = 0;
  for (int kb = k0; kb < k1; kb += 64 * kGroupUnroll) {
    stage(kb);
    const int nb = min(kGroupUnroll, (k1 - kb + 63) / 64);
#pragma unroll 1
    for (int u = 0; u < nb; ++u) {
      const int j = s_sj[wave][u * 64 + lane], e = s_se[wave][u * 64 + lane];
      uint32_t mm, mf;
      masks(j, e, kb + u * 64 + lane < k1, mm, mf);
      uint64_t runm = 0ull;
      const bool rstart = kw ? run_mask(j, runm) : false;
#pragma unroll
      for (int i = 0; i < kSuperTiles; ++i) {
        const bool member = (mm >> i) & 1u, full = (mf >> i) & 1u;
        const uint64_t bf = dma::ballot(full), bp = dma::ballot(member && !full);
        nfv += lane == i ? (int)__popcll(bf) : 0;
        npv += lane == i ? (int)__popcll(bp) : 0;
        if (rstart && ((bf | bp) & runm)) atomicOr(&s_kt[i * kw + (j >> 11)], 1u << ((j >> 6) & 31));
      }
    }
  }
  if (lane < kSuperTiles) {
    s_c[wave][lane][0] = nfv;
    s_c[wave][lane][1] = npv;
  }
  __syncthreads();
  // lane i: this wave's offsets in tile i's two runs
  int ofv = 0, opv = 0;
  if (lane < kSuperTiles) {
    int a = 0, bsum = 0, tf = 0, tp = 0;
    for (int w2 = 0; w2 < kGroupWaves; ++w2) {
      const int cf = s_c[w2][lane][0], cp = s_c[w2][lane][1];
      if (w2 < wave) {
        a += cf;
        bsum += cp;
      }
      tf += cf;
      tp += cp;
    }
    ofv = a;
    opv = tf + bsum;  // the partial run follows the full run
    if (wave == 0 && lane < ng) {
      const int64_t g = (int64_t)seg * n_tiles + t0 + lane;
      u_cnt[g] = min(tf + tp, u_stride);
      u_nfull[g] = min(tf, u_stride);
    }
  }
  int32_t* out0 = u_idx + ((int64_t)seg * n_tiles + t0) * u_stride;
  for (int kb = k0; kb < k1; kb += 64 * kGroupUnroll) {
    // a wave whose candidates fit one round still has them staged
    if (k1 - k0 > 64 * kGroupUnroll) stage(kb);
    const int nb = min(kGroupUnroll, (k1 - kb + 63) / 64);
#pragma unroll 1
    for (int u = 0; u < nb; ++u) {
      const int j = s_sj[wave][u * 64 + lane], e = s_se[wave][u * 64 + lane];
      uint32_t mm, mf;
      masks(j, e, kb + u * 64 + lane < k1, mm, mf);
#pragma unroll
      for (int i = 0; i < kSuperTiles; ++i) {
        const bool member = (mm >> i) & 1u, full = (mf >> i) & 1u;
        const uint64_t bf = dma::ballot(full), bp = dma::ballot(member && !full);
        const int of_i = __builtin_amdgcn_readlane(ofv, i), op_i = __builtin_amdgcn_readlane(opv, i);
        const int pos = full ? of_i + dma::rank_below(bf) : op_i + dma::rank_below(bp);
        if (member && pos < u_stride) out0[(int64_t)i * u_stride + pos] = j;
        ofv += lane == i ? (int)__popcll(bf) : 0;
        opv += lane == i ? (int)__popcll(bp) : 0;
      }
    }
  }
  if (kw) {
    __syncthreads();
    // one wave per tile: ordered compaction of its key-tile bitmap
    for (int i = wave; i < ng; i += kGroupWaves) {
      const uint32_t* bm = s_kt + i * kw;
      int32_t* kout = kt_idx + ((int64_t)seg * n_tiles + t0 + i) * kt_stride;
      int at = 0;
      for (int k = 0; k < kw; k += 64) {
        const uint32_t x = k + lane < kw ? bm[k + lane] : 0u;
        const int c = __popc(x);
        int incl = c;  // inclusive prefix over the wave
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int y = __shfl_up(incl, o);
          if (lane >= o) incl += y;
        }
        int pos = at + incl - c;
        uint32_t y = x;
        while (y) {
          const int b = __builtin_ctz(y);
          y &= y - 1;
          if (pos < kt_stride) kout[pos] = (k + lane) * 32 + b;
          ++pos;
        }
        at += __shfl(incl, 63);
      }
      if (lane == 0) kt_cnt[(int64_t)seg * n_tiles + t0 + i] = min(at, kt_stride);
    }
  }
}

// L1 + L2 in one workgroup per group, with the group's candidates held in
// LDS (when they fit: cap <= kFusedCap) instead of a round trip through
// global memory.  16 waves scan keys 0..P_hi for the candidates as L1 does,
// then build the tile lists from LDS as L2 does, each wave for a slice of
// the candidates and all tiles of the group: a counting pass (the tile
// masks stay in registers), one barrier for the offsets, a writing pass.
// Tile offsets are wave-uniform (scalar registers); list entries go out
// through a raw buffer view of the group's lists, lanes with nothing to
// store taking an offset past its end, so the stores need no branch; most
// members are full, so partial members are written only by the batches
// that hold any.  The largest deltas come from the sort's per-block maxima
// below the group and one 64-key segment per tile, one wave each.
constexpr int kFusedWaves = 16;
constexpr int kFusedCap = 8192;
constexpr int kFusedBatches = kFusedCap / (64 * kFusedWaves);  // 64-candidate batches per wave
constexpr uint32_t kBufferDrop = 0x40000000u;  // a store offset past any list region

__global__ __launch_bounds__(kFusedWaves * 64) void lists_kernel(
    const float* __restrict__ delta, const uint32_t* __restrict__ blk_code,
    const int32_t* __restrict__ evict, int Sk, int Sq, int q0, int n_super, int n_tiles, int cap,
    int u_stride, int kt_stride, int32_t* __restrict__ u_idx, int32_t* __restrict__ u_cnt,
    int32_t* __restrict__ u_nfull, float* __restrict__ u_dmax, float* __restrict__ u_dlo,
    int32_t* __restrict__ kt_idx, int32_t* __restrict__ kt_cnt) {
  extern __shared__ __align__(16) int32_t s_dyn[];
  int32_t* s_cj = s_dyn;             // [cap + 64] candidate keys, ascending (64 spill slots)
  int32_t* s_ce = s_dyn + cap + 64;  // [cap + 64] their eviction rows
  uint32_t* s_kt = reinterpret_cast<uint32_t*>(s_ce + cap + 64);  // per tile: key-tile bitmap
  __shared__ int s_cw[kFusedWaves];
  __shared__ int s_c[kFusedWaves][kSuperTiles][2];
  __shared__ uint32_t s_seg[kSuperTiles + 1];  // largest codes: below the group, per tile
  const int tid = threadIdx.x;
  const int seg = blockIdx.y, T = blockIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int t0 = T * kSuperTiles;
  const int ng = min(kSuperTiles, n_tiles - t0);  // tiles in this group
  const int P_lo = q0 + t0 * kListRows;
  const int P_hi = q0 + min(Sq, (T + 1) * kSuperTiles * kListRows) - 1;
  const int Pend = q0 + Sq - 1;  // last position
  const int kw = kt_idx ? (kt_stride + 31) / 32 : 0;
  for (int k = tid; k < ng * kw; k += kFusedWaves * 64) s_kt[k] = 0u;
  const float* Dl = delta + (int64_t)seg * Sk;

  // largest delta codes, loads issued first: wave i < ng the keys of tile
  // t0+i's own rows, the last wave the keys below P_lo (block maxima, then
  // the keys of the block holding P_lo)
  uint32_t dmx = 0u;
  if (wave < ng) {
    const int j = P_lo + 64 * wave + lane;
    dmx = j <= Pend ? dma::ord32(Dl[j]) : 0u;
  } else if (wave == kFusedWaves - 1) {
    const uint32_t* bc = blk_code + (int64_t)seg * ((Sk + 63) >> 6);
    const int nb0 = P_lo >> 6;
    for (int b = lane; b < nb0; b += 64) dmx = max(dmx, bc[b]);
    const int jp = (nb0 << 6) + lane;
    if (jp < P_lo) dmx = max(dmx, dma::ord32(Dl[jp]));
  }

  // ---- L1: the candidates C = { j <= P_hi : e_j > max(j, P_lo) }
  {
    const int32_t* E = evict + (int64_t)seg * Sk;
    const int n = P_hi + 1;
    const int L = ((n + 64 * kFusedWaves - 1) / (64 * kFusedWaves)) * 64;
    const int j0 = min(n, wave * L), j1 = min(n, j0 + L);
    // one load batch per wave (n <= 16384): the rows stay in registers across
    // the barrier; otherwise both passes load
    const bool one = L <= 64 * kListUnroll;
    int e[kListUnroll];
    auto load = [&](int jb) {
#pragma unroll
      for (int u = 0; u < kListUnroll; ++u) {
        const int j = jb + u * 64 + lane;
        e[u] = j < j1 ? E[j] : 0;
      }
    };
    int nc = 0;
    for (int jb = j0; jb < j1; jb += 64 * kListUnroll) {
      load(jb);
#pragma unroll
      for (int u = 0; u < kListUnroll; ++u) {
        const int j = jb + u * 64 + lane;
        nc += __popcll(dma::ballot(j < j1 && e[u] > max(j, P_lo)));
      }
    }
    if (lane == 0) s_cw[wave] = nc;
    if (wave < ng || wave == kFusedWaves - 1) {
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) dmx = max(dmx, (uint32_t)__shfl_xor((int)dmx, o));
      if (lane == 0) s_seg[wave < ng ? wave + 1 : 0] = dmx;
    }
    __syncthreads();
    int oc = 0;
#pragma unroll
    for (int k = 0; k < kFusedWaves; ++k)
      if (k < wave) oc += s_cw[k];
    for (int jb = j0; jb < j1; jb += 64 * kListUnroll) {
      if (!one) load(jb);
#pragma unroll
      for (int u = 0; u < kListUnroll; ++u) {
        const int j = jb + u * 64 + lane;
        const bool member = j < j1 && e[u] > max(j, P_lo);
        const uint64_t bm = dma::ballot(member);
        // non-members (and any overflow) write their own spill slot
        const int pos = oc + dma::rank_below(bm);
        const int at = (member && pos < cap) ? pos : cap + lane;
        s_cj[at] = j;
        s_ce[at] = e[u];
        oc += __popcll(bm);
      }
    }
  }
  __syncthreads();
  int nc = 0;
#pragma unroll
  for (int k = 0; k < kFusedWaves; ++k) nc += s_cw[k];
  nc = min(nc, cap);
  // tile t0+i: the largest delta over keys 0..p_hi (below the group and
  // tiles 0..i) and over the keys before its first row (below the group and
  // tiles 0..i-1; minus infinity when there are none: code 0)
  if (tid < ng) {
    auto value = [](uint32_t c) {  // inverse of ord32
      return c == 0u ? -INFINITY
                     : __uint_as_float((c & 0x80000000u) ? (c & 0x7fffffffu) : ~c);
    };
    uint32_t mlo = s_seg[0];
    for (int k = 1; k <= tid; ++k) mlo = max(mlo, s_seg[k]);
    u_dmax[(int64_t)seg * n_tiles + t0 + tid] = value(max(mlo, s_seg[tid + 1]));
    if (u_dlo) u_dlo[(int64_t)seg * n_tiles + t0 + tid] = value(mlo);
  }

  // ---- L2: member and full tile masks of a candidate (bit i: tile t0 + i),
  // in closed form: with r = j - P_lo, key j is in U of tile i iff e > j,
  // j <= Pend and floor(r/64) <= i <= floor((e-1-P_lo)/64); every row of
  // tile i keeps it iff also ceil(r/64) <= i and (e > Pend or
  // i <= floor((e-64-P_lo)/64)).  Packed: full bits, then partial bits << 8.
  auto span = [](int a, int b) -> uint32_t {  // bits a..b
    return (a > b || b < 0) ? 0u : (uint32_t)((2ull << b) - (1ull << a));
  };
  auto masks = [&](int j, int e, bool valid) -> uint32_t {
    const int r = j - P_lo;
    const bool any = valid && e > j && j <= Pend;
    const uint32_t mm = any ? span(r < 0 ? 0 : r >> 6, min((e - 1 - P_lo) >> 6, ng - 1)) : 0u;
    const int fb = e > Pend ? ng - 1 : min((e - 64 - P_lo) >> 6, ng - 1);
    const uint32_t mf = mm & span(r <= 0 ? 0 : (r + 63) >> 6, fb);
    return mf | ((mm & ~mf) << 8);
  };
  const int L2 = ((nc + 64 * kFusedWaves - 1) / (64 * kFusedWaves)) * 64;
  const int k0 = min(nc, wave * L2), k1 = min(nc, k0 + L2);
  int cF[kSuperTiles], cP[kSuperTiles];  // wave-uniform counts, then offsets
#pragma unroll
  for (int i = 0; i < kSuperTiles; ++i) cF[i] = cP[i] = 0;
  uint32_t pm[kFusedBatches];  // packed masks per batch
  int pj[kFusedBatches];       // keys per batch
#pragma unroll
  for (int bt = 0; bt < kFusedBatches; ++bt) {
    const int kb = k0 + 64 * bt;
    if (kb >= k1) break;
    const int kc = min(kb + lane, k1 - 1);
    pj[bt] = s_cj[kc];
    pm[bt] = masks(pj[bt], s_ce[kc], kb + lane < k1);
#pragma unroll
    for (int i = 0; i < kSuperTiles; ++i) {
      cF[i] += __popcll(dma::ballot((pm[bt] >> i) & 1u));
      cP[i] += __popcll(dma::ballot((pm[bt] >> (8 + i)) & 1u));
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < kSuperTiles; ++i) {
      s_c[wave][i][0] = cF[i];
      s_c[wave][i][1] = cP[i];
    }
  }
  __syncthreads();
  {
    // lane i: tile i's offsets for this wave (full run, then partial run)
    int of = 0, op = 0;
    if (lane < kSuperTiles) {
      int a = 0, bsum = 0, tf = 0, tp = 0;
      for (int w2 = 0; w2 < kFusedWaves; ++w2) {
        const int f = s_c[w2][lane][0], pc = s_c[w2][lane][1];
        if (w2 < wave) {
          a += f;
          bsum += pc;
        }
        tf += f;
        tp += pc;
      }
      of = a;
      op = tf + bsum;
      if (wave == 0 && lane < ng) {
        const int64_t g = (int64_t)seg * n_tiles + t0 + lane;
        u_cnt[g] = min(tf + tp, u_stride);
        u_nfull[g] = min(tf, u_stride);
      }
    }
#pragma unroll
    for (int i = 0; i < kSuperTiles; ++i) {
      cF[i] = __builtin_amdgcn_readlane(of, i);
      cP[i] = __builtin_amdgcn_readlane(op, i);
    }
  }
  // the group's lists: ng rows of u_stride entries
  const __amdgpu_buffer_rsrc_t lists = __builtin_amdgcn_make_buffer_rsrc(
      u_idx + ((int64_t)seg * n_tiles + t0) * u_stride, (short)0,
      (int)((uint32_t)ng * (uint32_t)u_stride * 4u), 0x00020000);
#pragma unroll
  for (int bt = 0; bt < kFusedBatches; ++bt) {
    const int kb = k0 + 64 * bt;
    if (kb >= k1) break;
    const int j = pj[bt];
    const uint32_t m = pm[bt];
#pragma unroll
    for (int i = 0; i < kSuperTiles; ++i) {
      const bool full = (m >> i) & 1u;
      const uint64_t bF = dma::ballot(full), bP = dma::ballot((m >> (8 + i)) & 1u);
      const int pf = __builtin_amdgcn_mbcnt_hi((uint32_t)(bF >> 32),
                                               __builtin_amdgcn_mbcnt_lo((uint32_t)bF, cF[i]));
      const bool okf = full && pf < u_stride;
      __builtin_amdgcn_raw_buffer_store_b32(
          (uint32_t)j, lists, okf ? (uint32_t)(i * u_stride + pf) * 4u : kBufferDrop, 0, 0);
      if (bP) {  // wave-uniform: batches with partial members are rare
        const bool part = (m >> (8 + i)) & 1u;
        const int pp = __builtin_amdgcn_mbcnt_hi((uint32_t)(bP >> 32),
                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)bP, cP[i]));
        const bool okp = part && pp < u_stride;
        __builtin_amdgcn_raw_buffer_store_b32(
            (uint32_t)j, lists, okp ? (uint32_t)(i * u_stride + pp) * 4u : kBufferDrop, 0, 0);
      }
      cF[i] += __popcll(bF);
      cP[i] += __popcll(bP);
    }
    if (kw) {
      // key tiles of the members: a lane marks its key tile for the tiles it
      // is a member of, unless the lane below (candidates ascend) is a member
      // of the same tile in the same key tile
      const uint32_t mm = (m | (m >> 8)) & 0xffu;
      const int ktl = j >> 6;
      const int vb = __shfl_up((ktl << 8) | (int)mm, 1);
      const uint32_t below = (lane > 0 && (vb >> 8) == ktl) ? (uint32_t)(vb & 0xff) : 0u;
      for (uint32_t mk = mm & ~below; mk; mk &= mk - 1u)
        atomicOr(&s_kt[__builtin_ctz(mk) * kw + (ktl >> 5)], 1u << (ktl & 31));
    }
  }
  if (kw) {
    __syncthreads();
    // one wave per tile: ordered compaction of its key-tile bitmap, four
    // bits per lane per round of 256 key tiles
    for (int t = wave; t < ng; t += kFusedWaves) {
      const uint32_t* bm = s_kt + t * kw;
      int32_t* kout = kt_idx + ((int64_t)seg * n_tiles + t0 + t) * kt_stride;
      int at = 0;
      for (int k = 0; k < kw; k += 8) {
        const int wi = k + (lane >> 3);
        const uint32_t nib = wi < kw ? (bm[wi] >> (4 * (lane & 7))) & 0xfu : 0u;
        const int c = __popc(nib);
        int incl = c;  // inclusive prefix over the wave
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int y = __shfl_up(incl, o);
          if (lane >= o) incl += y;
        }
        int pos = at + incl - c;
        const int base = wi * 32 + 4 * (lane & 7);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (((nib >> q) & 1u) && pos < kt_stride) kout[pos] = base + q;
          pos += (nib >> q) & 1u;
        }
        at += __shfl(incl, 63);
      }
      if (lane == 0) kt_cnt[(int64_t)seg * n_tiles + t0 + t] = min(at, kt_stride);
    }
  }
}

// ---------------------------------------------------------------- decode: one row
// Keys 0..p of one sequence; keeps the w best (Hugging Face blog "Trainable
// Dynamic Mask Sparse Attention", section "Mask Combination with Causal
// Constraints": the top w of the causally visible keys by delta, ties to the
// lower index).  One workgroup of 512 threads per sequence; thread t holds
// the weights of keys k*512 + t (coalesced loads, 64 registers; NaN past the
// row, which no comparison admits).  The kept set is every key above T, the
// w-th largest weight, plus the lowest-index keys equal to T, w keys in all.
//
// T comes from a bracket.  A sample of 512 keys (32 strata spread over the
// row, 16 keys from one 128-byte line in each, loaded ahead of the row so
// that it is processed while the row is still in flight) goes into 256 bins
// over its own range; the bins that hold the sample ranks a margin either
// side of the w-th largest's expected rank give bounds lo and hi.  As the
// row arrives, each thread counts its keys above hi and parks the weights in
// [lo, hi] in its own LDS column.  When fewer than w keys lie above hi, at
// least w at or above lo, and no column overflowed, T is found by 8-bit radix
// passes over the order codes of the parked weights (LDS histograms; every
// wave scans the bins itself, so one barrier per pass).  Otherwise (a row the
// sample misjudged, or heavy ties) the search runs bit by bit over every key:
// the leading kDecLead bits over all of them, the rest over the keys still in
// reach when there are at most kDecCand, else over all.
//
// The output is in index order: ballots turn the verdicts into one 64-bit
// word per 64-key tile (tile k*8 + wave from register k of wave `wave`), and
// thread t then owns tile t, which also gives the key-tile list.
constexpr int kDecThreads = 512;
constexpr int kDecWaves = kDecThreads / 64;
constexpr int kDecKPT = 64;          // rows up to 32768 keys
constexpr int kDecSlots = 24;        // parked bracket weights per thread
constexpr int kDecBins = 256;
constexpr int kDecPasses = 4;        // 8-bit radix passes cover 32 bits
constexpr int kDecLead = 12;         // bits fixed over the full set (fallback)
constexpr int kDecCand = 8192;       // candidates carried to the remaining bits (fallback)
constexpr int kDecCPT = kDecCand / kDecThreads;
static_assert(kDecSlots * kDecThreads >= kDecCand, "the fallback shares the slot array");
static_assert(kDecSlots * kDecThreads * 4 >= 2 * kDecThreads * 8, "the bitmaps reuse the slots");

// Barrier that waits for the wave's LDS accesses only: loads of the row that
// are still in flight stay in flight.  The empty asm statements keep the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void dec_lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));  // lgkmcnt(0) only
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Order code of a non-NaN float, a bijection onto [0x00800000, 0xff800000]
// with -0 and +0 one value: positive values map to u | 2^31, negative ones to
// -u (mod 2^32); 0 stays free for keys past the row.
__device__ __forceinline__ uint32_t dec_code(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u)) + (u >> 31);
}
constexpr uint32_t kCodeNegInf = 0x00800000u, kCodePosInf = 0xff800000u;
// the float of a code; codes below -inf's give -inf, above +inf's NaN (which
// no weight reaches)
__device__ __forceinline__ float dec_value(uint32_t c) {
  if (c <= kCodeNegInf) return -INFINITY;
  return __uint_as_float(c >= 0x80000000u ? c & 0x7fffffffu : 0u - c);
}

// DPP row shift right by S lanes inside 16-lane rows; lanes with no source
// get `fill`.
template <int S>
__device__ __forceinline__ int dec_shr(int x, int fill) {
  return __builtin_amdgcn_update_dpp(fill, x, 0x110 + S, 0xf, 0xf, false);
}
// Inclusive prefix sum over the wave: within rows by DPP shifts, then the
// row totals by readlane.
__device__ __forceinline__ int dec_wave_scan(int x) {
  x += dec_shr<1>(x, 0);
  x += dec_shr<2>(x, 0);
  x += dec_shr<4>(x, 0);
  x += dec_shr<8>(x, 0);
  const int t0 = __builtin_amdgcn_readlane(x, 15), t1 = __builtin_amdgcn_readlane(x, 31),
            t2 = __builtin_amdgcn_readlane(x, 47);
  const int row = (int)(threadIdx.x & 63) >> 4;
  return x + (row == 0 ? 0 : row == 1 ? t0 : row == 2 ? t0 + t1 : t0 + t1 + t2);
}
__device__ __forceinline__ uint32_t dec_wave_max(uint32_t x) {
  x = max(x, (uint32_t)dec_shr<1>((int)x, (int)x));
  x = max(x, (uint32_t)dec_shr<2>((int)x, (int)x));
  x = max(x, (uint32_t)dec_shr<4>((int)x, (int)x));
  x = max(x, (uint32_t)dec_shr<8>((int)x, (int)x));
  return max(max((uint32_t)__builtin_amdgcn_readlane((int)x, 15),
                 (uint32_t)__builtin_amdgcn_readlane((int)x, 31)),
             max((uint32_t)__builtin_amdgcn_readlane((int)x, 47),
                 (uint32_t)__builtin_amdgcn_readlane((int)x, 63)));
}
__device__ __forceinline__ uint32_t dec_wave_min(uint32_t x) {
  x = min(x, (uint32_t)dec_shr<1>((int)x, (int)x));
  x = min(x, (uint32_t)dec_shr<2>((int)x, (int)x));
  x = min(x, (uint32_t)dec_shr<4>((int)x, (int)x));
  x = min(x, (uint32_t)dec_shr<8>((int)x, (int)x));
  return min(min((uint32_t)__builtin_amdgcn_readlane((int)x, 15),
                 (uint32_t)__builtin_amdgcn_readlane((int)x, 31)),
             min((uint32_t)__builtin_amdgcn_readlane((int)x, 47),
                 (uint32_t)__builtin_amdgcn_readlane((int)x, 63)));
}

// Exclusive prefix sum over the 512 threads, total out; one barrier (LDS
// only: loads in flight stay in flight), so each call site needs its own s_w.
__device__ __forceinline__ int dec_scan512(int v, int* s_w, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = dec_wave_scan(v);
  if (lane == 63) s_w[wave] = incl;
  dec_lds_barrier();
  int before = 0;
  total = 0;
#pragma unroll
  for (int k = 0; k < kDecWaves; ++k) {
    const int t = s_w[k];
    if (k < wave) before += t;
    total += t;
  }
  return before + incl - v;
}

// Bins of an LDS histogram, larger values in higher bins: the bin b holding
// descending rank r (0-based), i.e. above(b) <= r < above(b) + h[b], where
// above(b) counts the entries of the bins past b.  Every wave computes it on
// its own from the same bins (lane l takes bins 252-4l .. 255-4l).  Returns
// -1 when r is past the total.
__device__ __forceinline__ int dec_find_bin(const uint32_t* hist, int r, int& above, int& inbin) {
  const int lane = threadIdx.x & 63;
  const uint4 h = reinterpret_cast<const uint4*>(hist)[63 - lane];
  const int s4 = (int)(h.x + h.y + h.z + h.w);
  int a = dec_wave_scan(s4) - s4;  // entries in the bins above this lane's
  int b = -1, ab = 0, hb = 0;
  const int hv[4] = {(int)h.w, (int)h.z, (int)h.y, (int)h.x};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (a <= r && r < a + hv[i]) {
      b = 255 - 4 * lane - i;
      ab = a;
      hb = hv[i];
    }
    a += hv[i];
  }
  const uint64_t m = dma::ballot(b >= 0);
  if (m == 0ull) {
    above = 0;
    inbin = 0;
    return -1;
  }
  const int src = __builtin_ctzll(m);
  above = __builtin_amdgcn_readlane(ab, src);
  inbin = __builtin_amdgcn_readlane(hb, src);
  return __builtin_amdgcn_readlane(b, src);
}

// Block total of per-thread counts in [0, 128) (fallback search): the wave
// sums its counts bit plane by bit plane with ballots (no cross-lane chains),
// one LDS slot per wave, one barrier.  Callers alternate two slot sets, which
// makes the one barrier enough: a wave cannot write a set again before every
// wave has passed the next call's barrier, i.e. finished reading it.
__device__ __forceinline__ int dec_block_count(int c, int* s_slots) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int tw = 0;
#pragma unroll
  for (int b = 0; b < 7; ++b) tw += __popcll(__ballot((c >> b) & 1)) << b;
  if (lane == 0) s_slots[wave] = tw;
  __syncthreads();
  int tot = 0;
#pragma unroll
  for (int v = 0; v < kDecWaves; ++v) tot += s_slots[v];
  return tot;
}

// One bit per round, hi down to lo: T | bit is taken when at least w keys
// reach it.  Over codes (0 for no key, below every candidate) or over the
// weights themselves (compared with the candidate's float; NaN past the row).
// cge tracks #{code >= T}.
__device__ __forceinline__ bool dec_reaches(uint32_t x, uint32_t cand, float) { return x >= cand; }
__device__ __forceinline__ bool dec_reaches(float x, uint32_t, float fc) { return x >= fc; }
__device__ __forceinline__ bool dec_above(uint32_t x, uint32_t T, float) { return x > T; }
__device__ __forceinline__ bool dec_above(float x, uint32_t, float fT) { return x > fT; }

template <typename X, int K>
__device__ __forceinline__ uint32_t dec_bit_search(const X (&x)[K], uint32_t T, int hi, int lo,
                                                   int w, int* s_cnt, int& round, int& cge) {
  for (int bit = hi; bit >= lo; --bit) {
    const uint32_t cand = T | (1u << bit);
    const float fc = dec_value(cand);
    int c = 0;
#pragma unroll
    for (int k = 0; k < K; ++k) c += dec_reaches(x[k], cand, fc) ? 1 : 0;
    const int tot = dec_block_count(c, s_cnt + (round & 1) * kDecWaves);
    ++round;
    if (tot >= w) {
      T = cand;
      cge = tot;
    }
  }
  return T;
}

template <typename X, int K>
__device__ __forceinline__ int dec_count_above(const X (&x)[K], uint32_t T, int* s_cnt,
                                               int& round) {
  const float fT = dec_value(T);
  int c = 0;
#pragma unroll
  for (int k = 0; k < K; ++k) c += dec_above(x[k], T, fT) ? 1 : 0;
  const int tot = dec_block_count(c, s_cnt + (round & 1) * kDecWaves);
  ++round;
  return tot;
}

__global__ __launch_bounds__(kDecThreads, 4) void decode_select_kernel(
    const float* __restrict__ delta, int Sk, int p, int w, int u_stride, int kt_stride,
    int32_t* __restrict__ u_idx, int32_t* __restrict__ u_cnt, int32_t* __restrict__ u_nfull,
    float* __restrict__ u_dmax, float* __restrict__ u_dval, int32_t* __restrict__ kt_idx,
    int32_t* __restrict__ kt_cnt) {
  __shared__ int s_w1[kDecWaves], s_w2[kDecWaves], s_w3[kDecWaves];
  __shared__ int s_cnt[2 * kDecWaves];
  __shared__ float s_m[kDecWaves];
  __shared__ uint32_t s_smin[kDecWaves], s_smax[kDecWaves];
  __shared__ int s_red[kDecWaves], s_ovf[kDecWaves];
  __shared__ __align__(16) uint32_t s_hist[kDecPasses + 1][kDecBins];
  // parked weights (thread t's column: entries t, t + 512, ...), then their
  // codes less lo; afterwards the tile bitmaps (weight >= T, or weight > T and
  // weight == T when ties are split)
  __shared__ __align__(16) uint32_t s_slots[kDecSlots * kDecThreads];
  uint32_t* const s_cand = s_slots;
  uint64_t* const s_gt = reinterpret_cast<uint64_t*>(s_slots);
  uint64_t* const s_eq = reinterpret_cast<uint64_t*>(s_slots) + kDecThreads;
  const int seg = blockIdx.x;
  const int n = p + 1;
  const float* Dl = delta + (int64_t)seg * Sk;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool sel = n > w;

  for (int i = tid; i < (kDecPasses + 1) * kDecBins; i += kDecThreads) (&s_hist[0][0])[i] = 0u;
  // The sample first, then the row.  Sample key of thread t: stratum t/16 of
  // 32 starts at a multiple of 32 keys near (t/16)*n/32, and takes every other
  // key of that 32-key line.  A relaxed atomic load is ordered, so it is
  // issued here rather than moved down to its use.
  const uint32_t skey =
      min((((uint32_t)(tid >> 4) * (uint32_t)n) >> 5 & ~31u) + 2u * (uint32_t)(tid & 15),
          (uint32_t)(n - 1));
  const float vs = __hip_atomic_load(Dl + skey, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  // register k: key k*512 + tid (past the row, a key of the last 512-key
  // block, loaded and then replaced by NaN); a wave-uniform block start plus
  // an offset below 512
  const int last = (n - 1) & ~(kDecThreads - 1);
  float v[kDecKPT];
#pragma unroll
  for (int k = 0; k < kDecKPT; ++k) {
    const int base = min(k * kDecThreads, last);
    v[k] = (Dl + base)[min((uint32_t)tid, (uint32_t)(n - 1 - base))];
  }
  const uint32_t sc = dec_code(vs);  // used here, so the load is not sunk into the branch

  // the bracket [lo, hi] as codes and as floats; with nothing to select it
  // admits no weight (NaN bounds)
  uint32_t lo = kCodeNegInf, hi = kCodePosInf;
  float flo = __uint_as_float(0x7fc00000u), fhi = flo;
  if (sel) {
    const uint32_t mn = dec_wave_min(sc), mxc = dec_wave_max(sc);
    if (lane == 0) {
      s_smin[wave] = mn;
      s_smax[wave] = mxc;
    }
    dec_lds_barrier();
    uint32_t gmin = s_smin[0], gmax = s_smax[0];
#pragma unroll
    for (int k = 1; k < kDecWaves; ++k) {
      gmin = min(gmin, s_smin[k]);
      gmax = max(gmax, s_smax[k]);
    }
    const uint32_t R = gmax - gmin;
    const int sh = R < (uint32_t)kDecBins ? 0 : 24 - __builtin_clz(R);
    const uint32_t dg = (sc - gmin) >> sh;  // < 256
    // a wave whose samples share one bin (a flat row) adds them at once
    const uint32_t d0 = __builtin_amdgcn_readfirstlane(dg);
    if (dma::ballot(dg != d0) == 0ull) {
      if (lane == 0) atomicAdd(&s_hist[0][d0], 64u);
    } else {
      atomicAdd(&s_hist[0][dg], 1u);
    }
    dec_lds_barrier();
    // expected descending sample rank of the w-th largest, and a margin of
    // about 4.5 binomial standard deviations either side
    const float q = (float)w / (float)n;
    const int margin = 4 + (int)(4.5f * sqrtf((float)kDecThreads * q * (1.f - q)));
    const int r = (int)(((int64_t)(2 * w - 1) * kDecThreads) / (2 * (int64_t)n));
    int ab, hb;
    if (r - margin >= 0) {
      const int b = dec_find_bin(s_hist[0], r - margin, ab, hb);
      if (b >= 0) {  // bin b's last code
        const uint64_t top = (uint64_t)gmin + ((uint64_t)(b + 1) << sh) - 1u;
        hi = (uint32_t)min(top, (uint64_t)kCodePosInf);
      }
    }
    if (r + margin < kDecThreads) {
      const int b = dec_find_bin(s_hist[0], r + margin, ab, hb);
      if (b >= 0) lo = max(gmin + ((uint32_t)b << sh), kCodeNegInf);  // bin b's first code
    }
    flo = dec_value(lo);
    fhi = dec_value(hi);
  }

  // the row: NaN past it, the largest weight, and the bracket pass
  float mx = -INFINITY;
  int c_gt = 0, c_in = 0;
#pragma unroll
  for (int k = 0; k < kDecKPT; ++k) {
    const float x = tid < n - k * kDecThreads ? v[k] : __uint_as_float(0x7fc00000u);
    v[k] = x;
    mx = fmaxf(mx, x);
    c_gt += x > fhi ? 1 : 0;
    if (x >= flo && x <= fhi) {
      if (c_in < kDecSlots) s_cand[c_in * kDecThreads + tid] = __float_as_uint(x);
      ++c_in;
    }
  }
  mx = dec_value(dec_wave_max(dec_code(mx)));  // max over codes: -0 and +0 as one
  if (lane == 0) s_m[wave] = mx;

  uint32_t T = kCodeNegInf;  // nothing to select: every key of the row
  int need_eq = 0;           // keys equal to T that are kept, lowest index first
  bool split = false;        // some keys equal to T are kept and some are not
  if (sel) {
    // block totals of c_gt and c_in (packed: each wave total is below 2^13)
    const int pk = __builtin_amdgcn_readlane(dec_wave_scan(c_gt | (c_in << 16)), 63);
    const bool ovf_w = dma::ballot(c_in > kDecSlots) != 0ull;
    if (lane == 0) {
      s_red[wave] = pk;
      s_ovf[wave] = ovf_w ? 1 : 0;
    }
    dec_lds_barrier();  // also publishes the parked weights
    int gt_hi = 0, n_in = 0, ovf = 0;
#pragma unroll
    for (int k = 0; k < kDecWaves; ++k) {
      const int x = s_red[k];
      gt_hi += x & 0xffff;
      n_in += x >> 16;
      ovf |= s_ovf[k];
    }
    if (!ovf && gt_hi < w && gt_hi + n_in >= w) {
      // radix passes over y = code - lo of the parked weights, 8 bits at a
      // time from the top bit of hi - lo down; need = the rank of T - lo
      // among them, from the top
      const uint32_t span = hi - lo;
      const int mine = min(c_in, kDecSlots);
      const int wmine = (int)dec_wave_max((uint32_t)mine);  // the wave's longest column
      uint32_t y[kDecSlots];
#pragma unroll
      for (int i = 0; i < kDecSlots; ++i) {
        if (i >= wmine) break;
        y[i] = i < mine ? dec_code(__uint_as_float(s_cand[i * kDecThreads + tid])) - lo : 0u;
      }
      int need = w - gt_hi, inb = n_in;
      int hbit = span == 0u ? 0 : 32 - __builtin_clz(span);
      uint32_t ypre = 0u;  // the bits of T - lo at and above hbit
      for (int pass = 0; pass < kDecPasses && hbit > 0; ++pass) {
        const int s = max(hbit - 8, 0);
        const uint32_t dmask = (1u << (hbit - s)) - 1u;
        // y matches the digits found so far: (y & hmask) == yfix
        const uint32_t hmask = hbit >= 32 ? 0u : ~0u << hbit;
        const uint32_t yfix = hbit >= 32 ? 0u : ypre << hbit;
        uint32_t* const hist = s_hist[1 + pass];
#pragma unroll
        for (int i = 0; i < kDecSlots; ++i) {
          if (i >= wmine) break;
          if (i < mine && (y[i] & hmask) == yfix) atomicAdd(&hist[(y[i] >> s) & dmask], 1u);
        }
        dec_lds_barrier();
        int above, inbin;
        const int d = dec_find_bin(hist, need - 1, above, inbin);
        need -= above;
        inb = inbin;
        ypre = (ypre << (hbit - s)) | (uint32_t)d;
        hbit = s;
      }
      T = lo + ypre;
      need_eq = need;
      split = need < inb;
    } else {
      int round = 0, cge = n;
      T = dec_bit_search(v, 0u, 31, 32 - kDecLead, w, s_cnt, round, cge);
      int gt_tot;
      if (cge <= kDecCand) {
        // order-free compaction of the codes of the keys at or above T
        const float fT = dec_value(T);
        int sc2 = 0;
#pragma unroll
        for (int k = 0; k < kDecKPT; ++k) sc2 += v[k] >= fT ? 1 : 0;
        int stot;
        int at = dec_scan512(sc2, s_w1, stot);
#pragma unroll
        for (int k = 0; k < kDecKPT; ++k)
          if (v[k] >= fT && at < kDecCand) s_cand[at++] = dec_code(v[k]);
        __syncthreads();
        uint32_t cr[kDecCPT];
#pragma unroll
        for (int i = 0; i < kDecCPT; ++i) {
          const int q = i * kDecThreads + tid;
          cr[i] = q < stot ? s_cand[q] : 0u;
        }
        T = dec_bit_search(cr, T, 31 - kDecLead, 0, w, s_cnt, round, cge);
        gt_tot = dec_count_above(cr, T, s_cnt, round);
      } else {
        T = dec_bit_search(v, T, 31 - kDecLead, 0, w, s_cnt, round, cge);
        gt_tot = dec_count_above(v, T, s_cnt, round);
      }
      need_eq = w - gt_tot;
      split = true;
    }
  }
  // tile bitmaps: the ballot of register k in wave `wave` is the word of key
  // tile k*8 + wave, stored at wave*64 + k (four registers per store group).
  // Every read of the parked weights is behind a barrier already passed.
  const float fT = dec_value(T);
  ulonglong2* const g2 = reinterpret_cast<ulonglong2*>(s_gt + wave * kDecKPT);
  ulonglong2* const e2 = reinterpret_cast<ulonglong2*>(s_eq + wave * kDecKPT);
  if (!split) {
#pragma unroll
    for (int k = 0; k < kDecKPT; k += 4) {
      const uint64_t a = dma::ballot(v[k] >= fT), b = dma::ballot(v[k + 1] >= fT);
      const uint64_t c = dma::ballot(v[k + 2] >= fT), d = dma::ballot(v[k + 3] >= fT);
      if (lane == 0) {
        g2[k / 2] = make_ulonglong2(a, b);
        g2[k / 2 + 1] = make_ulonglong2(c, d);
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < kDecKPT; k += 2) {
      const uint64_t a = dma::ballot(v[k] > fT), b = dma::ballot(v[k + 1] > fT);
      const uint64_t c = dma::ballot(v[k] == fT), d = dma::ballot(v[k + 1] == fT);
      if (lane == 0) {
        g2[k / 2] = make_ulonglong2(a, b);
        e2[k / 2] = make_ulonglong2(c, d);
      }
    }
  }
  __syncthreads();
  // thread t: keys [64t, 64t + 64), i.e. key tile t
  const int tw = (tid & (kDecWaves - 1)) * kDecKPT + (tid >> 3);
  uint64_t kept = s_gt[tw];
  if (split) {
    uint64_t x = s_eq[tw];
    const int ne = __popcll(x);
    int etot;
    const int eb = dec_scan512(ne, s_w2, etot);
    const int allow = min(ne, max(0, need_eq - eb));
    for (int r = 0; r < allow; ++r) {
      kept |= x & (~x + 1ull);
      x &= x - 1ull;
    }
  }
  int32_t* out = u_idx + (int64_t)seg * u_stride;
  float* dout = u_dval ? u_dval + (int64_t)seg * u_stride : nullptr;
  // the first kDecPre kept keys of the tile and their delta (cache hits: the
  // row was just read), loaded before the scan so that it hides the latency
  constexpr int kDecPre = 8;
  int pk[kDecPre];
  float pv[kDecPre];
  uint64_t rest = kept;
#pragma unroll
  for (int i = 0; i < kDecPre; ++i) {
    pk[i] = 64 * tid + (rest ? __builtin_ctzll(rest) : 0);  // key 64*tid: a real key
    rest &= rest - 1ull;
  }
  if (dout) {
#pragma unroll
    for (int i = 0; i < kDecPre; ++i) pv[i] = Dl[pk[i]];
  }
  // one scan for both the output offsets and the key-tile list (packed:
  // at most 32768 kept keys, 512 tiles)
  const int nk = __popcll(kept);
  const int f = kept != 0ull ? 1 : 0;
  int tot2;
  const int pre = dec_scan512(nk | (f << 16), s_w3, tot2);
  const int tot = tot2 & 0xffff, ktot = tot2 >> 16;
  int pos = pre & 0xffff;
#pragma unroll
  for (int i = 0; i < kDecPre; ++i) {
    if (i < nk && pos + i < u_stride) {
      out[pos + i] = pk[i];
      if (dout) dout[pos + i] = pv[i];
    }
  }
  pos += min(nk, kDecPre);
  for (uint64_t y = rest; y; y &= y - 1ull) {  // tiles with more kept keys
    if (pos < u_stride) {
      const int key = 64 * tid + __builtin_ctzll(y);
      out[pos] = key;
      if (dout) dout[pos] = Dl[key];
    }
    ++pos;
  }
  if (tid == 0) {
    float m = s_m[0];
    for (int k = 1; k < kDecWaves; ++k) m = fmaxf(m, s_m[k]);
    u_cnt[seg] = min(tot, u_stride);
    u_nfull[seg] = min(tot, u_stride);
    u_dmax[seg] = m;
  }
  if (kt_idx) {
    const int at = pre >> 16;
    if (f && at < kt_stride) kt_idx[(int64_t)seg * kt_stride + at] = tid;
    if (tid == 0) kt_cnt[seg] = min(ktot, kt_stride);
  }
}

// One row with more keys than decode_select_kernel holds in registers (the
// same selection: the w best of keys 0..p, ties to the lower index).  One
// workgroup of 1024 threads per sequence.  The threshold T, the w-th largest
// code, comes from four 8-bit radix passes over delta: each pass builds the
// histogram of the next digit among the keys whose leading digits match T's
// so far (per-wave LDS histograms; a wave whose matching lanes share one
// digit adds their count once), and a suffix scan picks the digit where the
// count of larger keys reaches w.  The output then takes the keys in index
// order in contiguous per-thread ranges of whole 64-key tiles: one pass
// counts the keys above T and equal to T per range, block scans give each
// range its share of the equal keys (lowest indices first) and its output
// offset, and a second pass writes the kept keys and the touched key tiles.
constexpr int kDecLThreads = 1024;
constexpr int kDecLWaves = kDecLThreads / 64;

// Exclusive prefix sum of v over the 1024 threads (two barriers); total out.
__device__ __forceinline__ int dec_block_scan(int v, int* s_w, int& total) {
  return block_excl_scan<kDecLThreads>(v, s_w, total);
}

__global__ __launch_bounds__(kDecLThreads) void decode_select_large_kernel(
    const float* __restrict__ delta, int Sk, int p, int w, int u_stride, int kt_stride,
    int32_t* __restrict__ u_idx, int32_t* __restrict__ u_cnt, int32_t* __restrict__ u_nfull,
    float* __restrict__ u_dmax, float* __restrict__ u_dval, int32_t* __restrict__ kt_idx,
    int32_t* __restrict__ kt_cnt) {
  __shared__ uint32_t s_hist[kDecLWaves][256];
  __shared__ int s_suf[257];
  __shared__ int s_w[kDecLWaves];
  __shared__ int s_sel[2];
  __shared__ float s_m[kDecLWaves];
  const int seg = blockIdx.x;
  const int n = p + 1;
  const float* Dl = delta + (int64_t)seg * Sk;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  uint32_t prefix = 0u, dmask = 0u;
  int above = 0;  // keys whose code exceeds every code with T's leading digits
  float mx = -INFINITY;
  const bool all = n <= w;
  for (int pass = 0; pass < 4 && !all; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int k = lane; k < 256; k += 64) s_hist[wave][k] = 0u;
    __syncthreads();
    for (int j0 = 0; j0 < n; j0 += kDecLThreads) {
      const int j = j0 + tid;
      const float v = j < n ? Dl[j] : 0.f;
      if (pass == 0 && j < n) mx = fmaxf(mx, v);
      const uint32_t c = dma::ord32(v);
      const bool m = j < n && (c & dmask) == prefix;
      const uint32_t dg = (c >> shift) & 255u;
      const uint64_t bm = dma::ballot(m);
      if (bm) {
        const int first = __builtin_ctzll(bm);
        const uint32_t d0 = (uint32_t)__shfl((int)dg, first);
        if (dma::ballot(m && dg == d0) == bm) {  // one digit for the whole wave
          if (lane == first) atomicAdd(&s_hist[wave][d0], (uint32_t)__popcll(bm));
        } else if (m) {
          atomicAdd(&s_hist[wave][dg], 1u);
        }
      }
    }
    __syncthreads();
    // suffix sums over the digits: s_suf[d] = keys with digit >= d
    if (tid < 256) {
      uint32_t t = 0u;
      for (int k = 0; k < kDecLWaves; ++k) t += s_hist[k][tid];
      s_suf[tid] = (int)t;
    }
    if (tid == 256) s_suf[256] = 0;
    __syncthreads();
    if (wave == 0) {
      // lane l: digits 4l..4l+3, then a suffix scan over the lanes
      int v4[4], tsum = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v4[q] = s_suf[4 * lane + q];
        tsum += v4[q];
      }
      int incl = tsum;  // inclusive suffix over lanes l..63
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_down(incl, o);
        if (lane + o < 64) incl += y;
      }
      int suf = incl - tsum;  // keys in digits above 4l+3
#pragma unroll
      for (int q = 3; q >= 0; --q) {
        const int hi = suf;  // digits above 4l+q
        suf += v4[q];
        if (above + suf >= w && above + hi < w) {
          s_sel[0] = 4 * lane + q;
          s_sel[1] = above + hi;
        }
      }
    }
    __syncthreads();
    prefix |= (uint32_t)s_sel[0] << shift;
    dmask |= 255u << shift;
    above = s_sel[1];
    __syncthreads();  // s_sel and the histograms are rewritten next pass
  }
  if (all) {
    for (int j0 = 0; j0 < n; j0 += kDecLThreads)
      if (j0 + tid < n) mx = fmaxf(mx, Dl[j0 + tid]);
  }
  const uint32_t T = prefix;
  const int need_eq = all ? 0 : w - above;  // keys equal to T that are kept, lowest index first

  // ranges of whole 64-key tiles, one per thread
  const int ntile = (n + 63) >> 6;
  const int tper = (ntile + kDecLThreads - 1) / kDecLThreads;
  const int k_lo = min(n, tid * tper * 64), k_hi = min(n, k_lo + tper * 64);
  int ng = 0, ne = 0;
  for (int j = k_lo; j < k_hi; ++j) {
    const uint32_t c = dma::ord32(Dl[j]);
    ng += (all || c > T) ? 1 : 0;
    ne += (!all && c == T) ? 1 : 0;
  }
  int tot;
  const int eb = dec_block_scan(ne, s_w, tot);  // equal keys before this range
  const int take = min(ne, max(0, need_eq - eb));
  int pos = dec_block_scan(ng + take, s_w, tot);
  int32_t* out = u_idx + (int64_t)seg * u_stride;
  float* dout = u_dval ? u_dval + (int64_t)seg * u_stride : nullptr;
  int kt_here = 0;
  {
    int eq_left = take;
    int last_tile = -1;
    for (int j = k_lo; j < k_hi; ++j) {
      const float dj = Dl[j];
      const uint32_t c = dma::ord32(dj);
      bool kept = all || c > T;
      if (!kept && c == T && eq_left > 0) {
        kept = true;
        --eq_left;
      }
      if (kept) {
        if (pos < u_stride) {
          out[pos] = j;
          if (dout) dout[pos] = dj;
        }
        ++pos;
        if ((j >> 6) != last_tile) {
          last_tile = j >> 6;
          ++kt_here;
        }
      }
    }
  }
  int ktot;
  int kpos = dec_block_scan(kt_here, s_w, ktot);
  if (kt_idx && kt_here) {
    int last_tile = -1, eq_left = take;
    for (int j = k_lo; j < k_hi; ++j) {
      const uint32_t c = dma::ord32(Dl[j]);
      bool kept = all || c > T;
      if (!kept && c == T && eq_left > 0) {
        kept = true;
        --eq_left;
      }
      if (kept && (j >> 6) != last_tile) {
        last_tile = j >> 6;
        if (kpos < kt_stride) kt_idx[(int64_t)seg * kt_stride + kpos] = last_tile;
        ++kpos;
      }
    }
  }
  mx = dma::wave_max(mx);
  if (lane == 0) s_m[wave] = mx;
  __syncthreads();
  if (tid == 0) {
    float m = s_m[0];
    for (int k = 1; k < kDecLWaves; ++k) m = fmaxf(m, s_m[k]);
    u_cnt[seg] = min(tot, u_stride);
    u_nfull[seg] = min(tot, u_stride);
    u_dmax[seg] = m;
    if (kt_idx) kt_cnt[seg] = min(ktot, kt_stride);
  }
}

// One decode step of the keep set (Hugging Face blog "Trainable Dynamic Mask
// Sparse Attention", section "Mask Combination with Causal Constraints": the
// keep set of position p is the top w of keys 0..p).  Because the sets nest,
// keep(p) is the top w of keep(p-1) plus key p: once keep(p-1) holds w keys,
// key p enters exactly when it beats the worst kept key, which it then
// replaces.  One workgroup per sequence: the w-entry ascending list goes to
// LDS, the worst entry (smallest 64-bit key) is found by a block reduction,
// and when key p enters the entries after the worst one shift down by one
// and p (the largest index) goes last.
constexpr int kAppThreads = 256;

__global__ __launch_bounds__(kAppThreads) void decode_append_kernel(
    const float* __restrict__ delta, int Sk, int w, int32_t* __restrict__ u_idx,
    int32_t* __restrict__ u_cnt, int32_t* __restrict__ u_nfull, float* __restrict__ u_dmax,
    float* __restrict__ u_dval) {
  extern __shared__ __align__(16) int32_t s_list[];  // [w]
  __shared__ uint64_t s_k[kAppThreads / 64];
  __shared__ float s_m[kAppThreads / 64];
  __shared__ int s_pos;
  const int seg = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* Dl = delta + (int64_t)seg * Sk;
  int32_t* list = u_idx + (int64_t)seg * w;
  if (u_cnt[seg] != w) return;  // keep(p-1) must be full: the caller's precondition
  const int p = Sk - 1;
  uint64_t kmin = ~0ull;
  int pmin = 0;
  float dmax = -INFINITY;
  for (int i = tid; i < w; i += kAppThreads) {
    const int j = list[i];
    s_list[i] = j;
    const float d = Dl[j];
    const uint64_t k = dma::key_of(d, (uint32_t)j);
    if (k < kmin) {
      kmin = k;
      pmin = i;
    }
    dmax = fmaxf(dmax, d);
  }
  // block minimum of the keys (all distinct) and maximum of delta
  uint64_t wk = kmin;
  float wm = dmax;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint64_t ok = ((uint64_t)(uint32_t)__shfl_xor((int)(wk >> 32), o) << 32) |
                        (uint32_t)__shfl_xor((int)(uint32_t)wk, o);
    wk = ok < wk ? ok : wk;
    wm = fmaxf(wm, __shfl_xor(wm, o));
  }
  if (lane == 0) {
    s_k[wave] = wk;
    s_m[wave] = wm;
  }
  __syncthreads();
  uint64_t gk = s_k[0];
  float gm = s_m[0];
  for (int k = 1; k < kAppThreads / 64; ++k) {
    gk = s_k[k] < gk ? s_k[k] : gk;
    gm = fmaxf(gm, s_m[k]);
  }
  if (kmin == gk) s_pos = pmin;  // exactly one thread holds the minimum
  __syncthreads();
  const float dp = Dl[p];
  const bool enters = dma::key_of(dp, (uint32_t)p) > gk;
  if (enters) {
    const int pm = s_pos;
    for (int i = pm + tid; i < w; i += kAppThreads) list[i] = i + 1 < w ? s_list[i + 1] : p;
  }
  if (u_dval) {  // every entry's delta, so no earlier state is assumed
    float* dl = u_dval + (int64_t)seg * w;
    const int pm = enters ? s_pos : w;
    for (int i = tid; i < w; i += kAppThreads)
      dl[i] = i < pm ? Dl[s_list[i]] : (i + 1 < w ? Dl[s_list[i + 1]] : dp);
  }
  if (tid == 0) {
    u_nfull[seg] = w;
    u_dmax[seg] = enters ? (w == 1 ? dp : fmaxf(gm, dp)) : gm;
  }
}

}  // namespace

// rank rows are padded to a multiple of 4 keys so each row starts 16-byte aligned
static int64_t rank_stride(int64_t Sk) { return (Sk + 3) & ~int64_t(3); }
static int64_t n_super_of(int64_t Sq) {
  const int64_t nt = (Sq + kListRows - 1) / kListRows;
  return (nt + kSuperTiles - 1) / kSuperTiles;
}
// candidates per tile group: keys kept at its first position plus keys born
// inside it, rounded up to whole 16-byte rows
static int64_t cand_cap(int64_t Sk, int64_t w) {
  const int64_t c = std::min<int64_t>(Sk, w + kSuperTiles * kListRows);
  return (c + 3) & ~int64_t(3);
}

// eviction checkpoints: every chk ranks (a multiple of 256), at most 64 per
// sequence
static int64_t ckpt_every(int64_t Sk) {
  const int64_t c = std::max<int64_t>(256, (Sk + 63) / 64);
  return (c + 255) & ~int64_t(255);
}
static int64_t ckpt_words(int64_t Sk) { return (((Sk + 31) >> 5) + 3) & ~int64_t(3); }

size_t dma_topk_ws_bytes(int64_t BH, int64_t Sq, int64_t Sk, int64_t w) {
  // two key buffers (ping-pong merges), ranks, the candidate lists, the
  // eviction checkpoints, then the largest delta code per 64-key block
  const size_t n = (size_t)BH * (size_t)Sk;
  const size_t ns = (size_t)BH * (size_t)n_super_of(Sq);
  const size_t nck = (size_t)BH * (size_t)((Sk + ckpt_every(Sk) - 1) / ckpt_every(Sk));
  return n * 2 * sizeof(uint64_t) + (size_t)BH * rank_stride(Sk) * sizeof(int32_t) +
         ns * (size_t)cand_cap(Sk, w) * 8 + ns * sizeof(int32_t) +
         nck * (size_t)ckpt_words(Sk) * sizeof(uint32_t) +
         (size_t)BH * (size_t)((Sk + 63) / 64) * sizeof(uint32_t) + 256;
}

// Scratch for callers that cannot allocate (dma_topk_mask_noalloc): the
// prefill mask workspace in a static device array, one per GPU, held until
// the process ends.  Host code must not pass `scratch` itself to a kernel
// (that names a host-side stand-in): each device's address comes from
// hipGetSymbolAddress, taken once per device with that device current.
static __device__ __align__(256) unsigned char scratch[DMA_TOPK_SCRATCH_BYTES];

hipError_t dma_topk_scratch(void** ptr) {
  constexpr int kMaxDev = 64;
  static void* addr[kMaxDev] = {nullptr};
  static std::mutex mu;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t dma_launch_topk_prefill(const DmaTopkArgs& a, hipStream_t st) {
  const int64_t BH = a.B * a.Hkv;
  const int Sk = (int)a.Sk;
  const size_t n = (size_t)BH * (size_t)Sk;
  uint64_t* kA = static_cast<uint64_t*>(a.ws);
  uint64_t* kB = kA + n;
  int32_t* rank = reinterpret_cast<int32_t*>(kB + n);
  const int rs = (int)rank_stride(Sk);
  const int n_super = (int)n_super_of(a.Sq);
  const int cap = (int)cand_cap(a.Sk, a.w);
  int32_t* cj = rank + BH * rs;
  int32_t* ce = cj + (size_t)BH * n_super * cap;
  int32_t* ccnt = ce + (size_t)BH * n_super * cap;
  uint32_t* ckpt = reinterpret_cast<uint32_t*>(ccnt + (size_t)BH * n_super);
  const int chk = (int)ckpt_every(Sk);
  const int n_chk = (Sk + chk - 1) / chk;
  const int nwr = (int)ckpt_words(Sk);
  const size_t bm_bytes = (size_t)nwr * sizeof(uint32_t);
  uint32_t* blk = ckpt + (size_t)BH * n_chk * nwr;

  // up to kRankRunsMax small runs: ranks by binary search; beyond that,
  // large runs and merges
  const bool by_search = Sk > kSortChunkSmall && Sk <= kRankRunsMax * kSortChunkSmall;
  const int chunk = by_search || Sk <= kSortChunkSmall ? kSortChunkSmall : kSortChunkLarge;
  const int nch = (Sk + chunk - 1) / chunk;
  // runs for the binary searches: codes and reversed-index bits, rows of
  // cstride entries, in the first key buffer
  const int cstride = (Sk + 7) & ~7;
  uint32_t* rcodes = reinterpret_cast<uint32_t*>(kA);
  uint16_t* rrevs = reinterpret_cast<uint16_t*>(rcodes + (size_t)BH * cstride);
  if (by_search)
    hipLaunchKernelGGL((sort_chunk_kernel<kSortChunkSmall, true>), dim3(nch, BH),
                       dim3(kSortChunkSmall / kSortPer), 0, st, a.delta, Sk, kA, rcodes, rrevs,
                       cstride, blk);
  else if (chunk == kSortChunkSmall)
    hipLaunchKernelGGL((sort_chunk_kernel<kSortChunkSmall, false>), dim3(nch, BH),
                       dim3(kSortChunkSmall / kSortPer), 0, st, a.delta, Sk, kA, rcodes, rrevs,
                       cstride, blk);
  else
    hipLaunchKernelGGL((sort_chunk_kernel<kSortChunkLarge, false>), dim3(nch, BH),
                       dim3(kSortChunkLarge / kSortPer), 0, st, a.delta, Sk, kA, rcodes, rrevs,
                       cstride, blk);
  uint64_t* src = kA;
  uint64_t* dst = kB;
  if (by_search) {
    // one dimension, sequence fastest
    const dim3 grid(nch * (kSortChunkSmall / kRankRunsKeys) * BH);
    auto launch = [&](auto kern, int nr) {
      const size_t lds = (size_t)nr * kSortChunkSmall * (sizeof(uint32_t) + sizeof(uint16_t));
      (void)dma_func_max_lds(reinterpret_cast<const void*>(kern), lds);
      hipLaunchKernelGGL(kern, grid, dim3(kRankRunsThreads), lds, st, rcodes, rrevs, cstride, Sk,
                         rs, rank, dst, (int)BH);
    };
    if (nch <= 4) launch(rank_runs_kernel<4>, 4);
    else if (nch <= 8) launch(rank_runs_kernel<8>, 8);
    else launch(rank_runs_kernel<16>, 16);
    src = dst;
  } else {
    for (int L = chunk; L < Sk; L <<= 1) {
      const int nthr = (Sk + kMergeItems - 1) / kMergeItems;
      hipLaunchKernelGGL(merge_kernel, dim3((nthr + 255) / 256, BH), dim3(256), 0, st, src, dst,
                         Sk, L);
      uint64_t* t = src;
      src = dst;
      dst = t;
    }
    hipLaunchKernelGGL(rank_kernel, dim3((Sk + 255) / 256, BH), dim3(256), 0, st, src, Sk, rs,
                       rank);
  }
  // eviction rows: 256-rank workgroups up to 16384 keys (checkpoints every
  // 256 ranks: the base bitmap is one checkpoint; per wave a bitmap and its
  // word prefixes in LDS), else 64-rank workgroups
  const size_t wg_lds = (size_t)(1 + 2 * kEvictWG) * bm_bytes + (size_t)kEvictRanks * sizeof(int);
  if (n_chk > 1)
    hipLaunchKernelGGL(ckpt_kernel, dim3((nwr * 32 + 255) / 256, BH), dim3(256), 0, st, rank, Sk,
                       rs, chk, n_chk, nwr, ckpt);
  if (chk == kEvictRanks) {
    (void)dma_func_max_lds(reinterpret_cast<const void*>(&evict_wg_kernel), wg_lds);
    hipLaunchKernelGGL(evict_wg_kernel, dim3((Sk + kEvictRanks - 1) / kEvictRanks, BH),
                       dim3(kEvictRanks), wg_lds, st, src, Sk, (int)a.w, chk, n_chk, nwr, ckpt,
                       a.evict);
  } else {
    const size_t ev_lds = bm_bytes + (8 + 64) * sizeof(int);  // bitmap, s_w[8], s_m[64]
    (void)dma_func_max_lds(reinterpret_cast<const void*>(&evict_kernel), ev_lds);
    hipLaunchKernelGGL(evict_kernel, dim3((Sk + kEvictR - 1) / kEvictR, BH), dim3(kEvictThreads),
                       ev_lds, st, src, Sk, (int)a.w, chk, n_chk, nwr, ckpt, a.evict);
  }
  const int kwords = a.kt_idx ? (int)((a.kt_stride + 31) / 32) : 0;
  if (kwords > kMaxKtWords) return hipErrorInvalidValue;
  if (cap <= kFusedCap) {
    const size_t lds = (size_t)2 * (cap + 64) * sizeof(int32_t) +
                       (size_t)kSuperTiles * kwords * sizeof(uint32_t);
    (void)dma_func_max_lds(reinterpret_cast<const void*>(&lists_kernel), lds);
    hipLaunchKernelGGL(lists_kernel, dim3(n_super, BH), dim3(kFusedWaves * 64), lds, st, a.delta,
                       blk, a.evict, Sk, (int)a.Sq, (int)a.q0, n_super, (int)a.n_tiles, cap,
                       (int)a.u_stride, (int)a.kt_stride, a.u_idx, a.u_cnt, a.u_nfull, a.u_dmax,
                       a.u_dlo, a.kt_idx, a.kt_cnt);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(cand_kernel, dim3(n_super, BH), dim3(kListWaves * 64), 0, st, a.delta,
                     a.evict, Sk, (int)a.Sq, (int)a.q0, n_super, (int)a.n_tiles, cap, cj, ce, ccnt,
                     a.u_dmax, a.u_dlo);
  const size_t kt_lds = (size_t)kSuperTiles * kwords * sizeof(uint32_t);
  if (kt_lds > 0)
    (void)dma_func_max_lds(reinterpret_cast<const void*>(&group_lists_kernel), kt_lds);
  hipLaunchKernelGGL(group_lists_kernel, dim3(n_super, BH), dim3(kGroupWaves * 64), kt_lds, st,
                     cj, ce, ccnt, (int)a.Sq, (int)a.q0, (int)a.n_tiles, n_super, cap,
                     (int)a.u_stride, (int)a.kt_stride, a.u_idx, a.u_cnt, a.u_nfull, a.kt_idx,
                     a.kt_cnt);
  return hipGetLastError();
}

void dma_cand_dims(int64_t Sq, int64_t Sk, int64_t w, int64_t* n_super, int64_t* cap) {
  *n_super = n_super_of(Sq);
  *cap = cand_cap(Sk, w);
}

hipError_t dma_launch_cand(const float* delta, const int32_t* evict, int64_t BH, int64_t Sk,
                           int64_t Sq, int64_t q0, int64_t w, int32_t* cj, int32_t* ce,
                           int32_t* ccnt, float* tile_dmax, hipStream_t st) {
  const int n_super = (int)n_super_of(Sq);
  const int cap = (int)cand_cap(Sk, w);
  const int n_tiles = (int)((Sq + kListRows - 1) / kListRows);
  hipLaunchKernelGGL(cand_kernel, dim3(n_super, (unsigned)BH), dim3(kListWaves * 64), 0, st,
                     delta, evict, (int)Sk, (int)Sq, (int)q0, n_super, n_tiles, cap, cj, ce, ccnt,
                     tile_dmax, (float*)nullptr);
  return hipGetLastError();
}

hipError_t dma_launch_decode_append(const float* delta, int64_t BH, int64_t Sk, int64_t w,
                                   int32_t* u_idx, int32_t* u_cnt, int32_t* u_nfull,
                                   float* u_dmax, float* u_dval, hipStream_t st) {
  const size_t lds = (size_t)w * sizeof(int32_t);
  (void)dma_func_max_lds(reinterpret_cast<const void*>(&decode_append_kernel), lds);
  hipLaunchKernelGGL(decode_append_kernel, dim3((unsigned)BH), dim3(kAppThreads), lds, st, delta,
                     (int)Sk, (int)w, u_idx, u_cnt, u_nfull, u_dmax, u_dval);
  return hipGetLastError();
}

hipError_t dma_launch_topk_decode(const DmaTopkArgs& a, hipStream_t st) {
  const int64_t BH = a.B * a.Hkv;
  if (a.q0 + 1 <= kDecThreads * kDecKPT)
    hipLaunchKernelGGL(decode_select_kernel, dim3(BH), dim3(kDecThreads), 0, st, a.delta,
                       (int)a.Sk, (int)a.q0, (int)a.w, (int)a.u_stride, (int)a.kt_stride, a.u_idx,
                       a.u_cnt, a.u_nfull, a.u_dmax, a.u_dval, a.kt_idx, a.kt_cnt);
  else
    hipLaunchKernelGGL(decode_select_large_kernel, dim3(BH), dim3(kDecLThreads), 0, st, a.delta,
                       (int)a.Sk, (int)a.q0, (int)a.w, (int)a.u_stride, (int)a.kt_stride, a.u_idx,
                       a.u_cnt, a.u_nfull, a.u_dmax, a.u_dval, a.kt_idx, a.kt_cnt);
  return hipGetLastError();
}
