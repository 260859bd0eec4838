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
//       bitonic sort of 4096-key chunks (registers, lane shuffles and LDS),
//       then merge-path merges;
//   T1b rank[j] = position of key j in that order; up to four chunks skip the
//       merges: a key's rank is the sum over the chunks of the keys that beat
//       it, found by binary searches over the chunks held in LDS;
//   T2  eviction rows: ranks are cut into blocks of 64; a block builds the
//       bitmap of the indices of all better-ranked keys (a checkpoint bitmap
//       kept every 1024 ranks plus the keys in between), selects its w-th
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

#include <algorithm>
#include <climits>

namespace {

constexpr int kSortChunk = 4096;
#ifndef DMA_SORT_PER
#define DMA_SORT_PER 4
#endif
constexpr int kSortPer = DMA_SORT_PER;  // keys per thread: element i = thread * kSortPer + register
constexpr int kSortThreads = kSortChunk / kSortPer;
constexpr int kSortRegBits = kSortPer == 8 ? 3 : kSortPer == 4 ? 2 : 4;
constexpr int kMergeItems = 8;
constexpr int kListRows = 64;   // query rows per tile (Bq)

// ---------------------------------------------------------------- T1: chunk sort
__device__ __forceinline__ uint64_t shfl_xor64(uint64_t v, int m) {
  const int lo = __shfl_xor((int)(uint32_t)v, m);
  const int hi = __shfl_xor((int)(uint32_t)(v >> 32), m);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

// Bitonic sort (descending) of a 4096-key chunk, in the form whose comparators
// all point one way: phase k (block size 2, 4, ..., 4096) first pairs i with
// its mirror i ^ (k-1) in the block, then with i ^ j for j = k/4, ..., 1, and
// the lower index of every pair keeps the larger key.  Element i lives in
// register i%8 of thread i/8, so pairs at distance < 8 stay inside a thread,
// pairs that differ in bits 3..8 pair lanes of one wave, and only pairs that
// differ in bits 9..11 cross waves, through LDS (two buffers, one barrier
// each).  Every element is updated by its owner, which takes the larger or the
// smaller of itself and its partner.
__global__ __launch_bounds__(kSortThreads) void sort_chunk_kernel(const float* __restrict__ delta,
                                                                  int Sk,
                                                                  uint64_t* __restrict__ out) {
  __shared__ uint64_t s[2][kSortChunk];
  const int seg = blockIdx.y;
  const int c0 = blockIdx.x * kSortChunk;
  const int lane = threadIdx.x & 63;
  const int base = threadIdx.x * kSortPer;
  const float* d = delta + (int64_t)seg * Sk;
  uint64_t a[kSortPer];
#pragma unroll
  for (int r = 0; r < kSortPer; ++r) {
    const int j = c0 + base + r;
    a[r] = (j < Sk) ? dma::key_of(d[j], (uint32_t)j) : 0ull;  // 0 sorts after every real key
  }
  int lds_stage = 0;  // LDS stages alternate buffers, so a buffer is rewritten
                      // only after the barrier of the stage in between
#pragma unroll
  for (int m = 1; m <= 12; ++m) {
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
        for (int r = 0; r < kSortPer; ++r) p[r] = shfl_xor64(a[r ^ (x & (kSortPer - 1))], lm);
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
  uint64_t* o = out + (int64_t)seg * Sk;
#pragma unroll
  for (int r = 0; r < kSortPer; ++r)
    if (c0 + base + r < Sk) o[c0 + base + r] = a[r];
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

// T1 + T1b for a sequence of at most four sorted 4096-key runs (up to 16K
// keys), in place of the merges: the rank of a key is its position in its own
// run plus, for each other run, the number of keys there that beat it (keys
// are distinct, so this is a binary search).  A workgroup holds every run of
// its sequence in LDS and ranks the keys of one run; it writes rank[j] and
// the merged order.
constexpr int kRankRunsMax = 4;
constexpr int kRankRunsThreads = 256;
constexpr int kRankRunsKeys = 1024;   // keys ranked per workgroup

__global__ __launch_bounds__(kRankRunsThreads) void rank_runs_kernel(
    const uint64_t* __restrict__ runs, int Sk, int rstride, int32_t* __restrict__ rank,
    uint64_t* __restrict__ merged) {
  extern __shared__ __align__(16) uint64_t s_runs[];
  const int seg = blockIdx.y;
  const int nr = (Sk + kSortChunk - 1) / kSortChunk;
  const uint64_t* src = runs + (int64_t)seg * Sk;
  // all runs of the sequence into LDS; a sequence starts 8-byte aligned only
  // (odd Sk), so 8-byte loads, all of a thread's in flight at once
  constexpr int kFill = kRankRunsMax * kSortChunk / kRankRunsThreads;
  for (int i0 = threadIdx.x; i0 < Sk; i0 += kRankRunsThreads * kFill) {
    uint64_t v[kFill];
#pragma unroll
    for (int u = 0; u < kFill; ++u) v[u] = src[min(i0 + u * kRankRunsThreads, Sk - 1)];
#pragma unroll
    for (int u = 0; u < kFill; ++u)
      if (i0 + u * kRankRunsThreads < Sk) s_runs[i0 + u * kRankRunsThreads] = v[u];
  }
  __syncthreads();

  // rank = sum over all runs (its own included, where the count is its
  // position) of the keys that beat it; the 4 keys x 4 runs searches of a
  // thread advance together, one halving step at a time
  constexpr int kU = kRankRunsKeys / kRankRunsThreads;
  const int r = blockIdx.x / (kSortChunk / kRankRunsKeys);
  const int q0 = (blockIdx.x % (kSortChunk / kRankRunsKeys)) * kRankRunsKeys + threadIdx.x;
  const int len_r = min(kSortChunk, Sk - r * kSortChunk);
  uint64_t x[kU];
  int cnt[kU][kRankRunsMax];
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    x[u] = s_runs[r * kSortChunk + min(q0 + u * kRankRunsThreads, len_r - 1)];
#pragma unroll
    for (int o = 0; o < kRankRunsMax; ++o) cnt[u][o] = 0;
  }
#pragma unroll
  for (int step = kSortChunk; step > 0; step >>= 1) {
#pragma unroll
    for (int o = 0; o < kRankRunsMax; ++o) {
      // no branch on the run count, so all 16 reads of a step are in flight
      // together; a missing run (n = 0) reads key 0 and never counts
      const int n = o < nr ? min(kSortChunk, Sk - o * kSortChunk) : 0;
      const uint64_t* A = s_runs + (o < nr ? o * kSortChunk : 0);
      uint64_t v[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) v[u] = A[max(min(cnt[u][o] + step, n), 1) - 1];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int i = cnt[u][o] + step;
        cnt[u][o] = (i <= n && v[u] > x[u]) ? i : cnt[u][o];
      }
    }
  }
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    if (q0 + u * kRankRunsThreads >= len_r) continue;
    int pos = 0;
#pragma unroll
    for (int o = 0; o < kRankRunsMax; ++o) pos += cnt[u][o];
    rank[(int64_t)seg * rstride + dma::index_of(x[u])] = pos;
    merged[(int64_t)seg * Sk + pos] = x[u];
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
// Bitmap of { j : rank[j] < rs } over nw 32-bit words in LDS: thread t
// builds words [t*per, (t+1)*per) from its contiguous ranks with 16-byte
// loads (unconditional, clamped into the sequence's padded rank row, so they
// all issue before the first is used; indices >= Sk are masked).
template <int NT>
__device__ __forceinline__ void rank_bitmap(const int32_t* __restrict__ rk, int Sk, int rstride,
                                            int rs, int nw, uint32_t* bm) {
  const int per = (nw + NT - 1) / NT;
  const int wlo = min(nw, (int)threadIdx.x * per), whi = min(nw, wlo + per);
  const int jmax = rstride - 4;
  for (int wi = wlo; wi < whi; wi += 2) {
    uint32_t word[2] = {0u, 0u};
    int4 v[2][8];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int q = 0; q < 8; ++q)
        v[u][q] = *reinterpret_cast<const int4*>(rk + min((wi + u) * 32 + q * 4, jmax));
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int j = (wi + u) * 32 + q * 4;
        word[u] |= (j < Sk && v[u][q].x < rs ? 1u : 0u) << (q * 4);
        word[u] |= (j + 1 < Sk && v[u][q].y < rs ? 1u : 0u) << (q * 4 + 1);
        word[u] |= (j + 2 < Sk && v[u][q].z < rs ? 1u : 0u) << (q * 4 + 2);
        word[u] |= (j + 3 < Sk && v[u][q].w < rs ? 1u : 0u) << (q * 4 + 3);
      }
      if (wi + u < whi) bm[wi + u] = word[u];
    }
  }
}

// T2a: checkpoint bitmaps { j : rank[j] < c * chk } for c = 1 .. n_chk-1,
// nwr words each, so an eviction block needs at most chk-1 insertions.
__global__ __launch_bounds__(256) void ckpt_kernel(const int32_t* __restrict__ rank, int Sk,
                                                   int rstride, int chk, int n_chk, int nwr,
                                                   uint32_t* __restrict__ ckpt) {
  extern __shared__ __align__(16) uint32_t bm[];
  const int seg = blockIdx.y, c = blockIdx.x + 1;
  const int nw = (Sk + 31) >> 5;
  rank_bitmap<256>(rank + (int64_t)seg * rstride, Sk, rstride, c * chk, nw, bm);
  __syncthreads();
  uint32_t* out = ckpt + ((int64_t)seg * n_chk + c) * nwr;
  for (int k = threadIdx.x; k < nwr; k += 256) out[k] = k < nw ? bm[k] : 0u;
}

// T2b: eviction rows of the keys of ranks [r0, r0 + R), one wave walking them.
__global__ __launch_bounds__(256) void evict_kernel(const uint64_t* __restrict__ sorted, int Sk,
                                                    int w, int R, int chk, int n_chk, int nwr,
                                                    const uint32_t* __restrict__ ckpt,
                                                    int32_t* __restrict__ evict) {
  // Dynamic LDS only, so the bitmap starts at byte 0 (8-byte aligned for the
  // 64-bit word reads): bitmap of indices in whole 64-bit words, then s_w, s_f.
  extern __shared__ __align__(16) uint32_t bm[];
  int* s_w = reinterpret_cast<int*>(bm + nwr);
  int& s_f = s_w[4];
  const int seg = blockIdx.y;
  const uint64_t* K = sorted + (int64_t)seg * Sk;
  int32_t* E = evict + (int64_t)seg * Sk;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r0 = blockIdx.x * R, r1 = min(Sk, r0 + R);
  // the w best keys are never beaten by w others: kept to the end
  for (int r = r0 + (int)threadIdx.x; r < min(r1, w); r += 256) E[dma::index_of(K[r])] = Sk;
  const int rs = max(r0, w);
  if (rs >= r1) return;

  // Bitmap of { j : rank[j] < rs }: the nearest checkpoint below rs, then
  // the keys of the ranks in between, then the w-th smallest set bit from
  // per-thread popcounts and one block scan.
  const int c = rs / chk;
  const uint32_t* cp = ckpt + ((int64_t)seg * n_chk + c) * nwr;
  for (int k = threadIdx.x; k < nwr; k += 256) bm[k] = c > 0 ? cp[k] : 0u;
  __syncthreads();
  for (int r = c * chk + (int)threadIdx.x; r < rs; r += 256) {
    const uint32_t x = dma::index_of(K[r]);
    atomicOr(&bm[x >> 5], 1u << (x & 31));
  }
  __syncthreads();
  const int nw = (Sk + 31) >> 5;
  const int per = (nw + 255) / 256;
  const int wlo = min(nw, (int)threadIdx.x * per), whi = min(nw, wlo + per);
  int cnt = 0;
  for (int k = wlo; k < whi; ++k) cnt += __popc(bm[k]);
  int total;
  const int before = block_excl_scan<256>(cnt, s_w, total);
  if (threadIdx.x == 0 && total < w) s_f = -1;  // unreachable: rs >= w ranks are set
  if (before < w && before + cnt >= w) {
    int need = w - before;
    for (int k = wlo; k < whi; ++k) {
      uint32_t x = bm[k];
      const int cc = __popc(x);
      if (need <= cc) {
        for (int q = 1; q < need; ++q) x &= x - 1;
        s_f = k * 32 + __builtin_ctz(x);
        break;
      }
      need -= cc;
    }
  }
  __syncthreads();
  if (wave != 0) return;

  // Walk the block's ranks in order on one wave.  Everything the walk carries
  // is wave-uniform (scalar registers): f, the 64-bit bitmap word holding f
  // and the word below it (both with this walk's own insertions), and f's
  // word index.  Insertions further down go to LDS, which is read again only
  // when f gets there; f only ever moves down.  Per 64 keys, a ballot of
  // x < f picks the keys that can move f (f only decreases, so no other key
  // can); they are visited in order and the others keep e = x.
  uint64_t* bm64 = reinterpret_cast<uint64_t*>(bm);
  int f = s_f;
  if (f < 0) return;  // unreachable (see above)
  int cwi = f >> 6;
  uint64_t cw = bm64[cwi];
  uint64_t pw = cwi > 0 ? bm64[cwi - 1] : 0ull;
  for (int g0 = rs; g0 < r1; g0 += 64) {
    const int steps = min(64, r1 - g0);
    const int xl = lane < steps ? (int)dma::index_of(K[g0 + lane]) : INT_MAX;  // one key per lane
    int el = xl;  // e = x unless the key moves f
    uint64_t cand = dma::ballot(xl < f);
    while (cand) {
      const int sl = __builtin_ctzll(cand);
      cand &= cand - 1ull;
      const int x = __builtin_amdgcn_readlane(xl, sl);
      if (x < f) {
        el = lane == sl ? f : el;  // e = f for this key
        const int xw = x >> 6;
        const uint64_t bit = 1ull << (x & 63);
        if (xw == cwi) {
          cw |= bit;
        } else if (xw == cwi - 1) {
          pw |= bit;
        } else if (lane == 0) {
          atomicOr(&bm[x >> 5], 1u << (x & 31));  // ds_or_b32: no return, no wait
        }
        // f <- largest set index below f (x itself qualifies)
        uint64_t m = cw & ((1ull << (f & 63)) - 1ull);
        if (m == 0ull) {
          cw = pw;
          --cwi;
          m = cw;
          while (m == 0ull && cwi > 0) {
            --cwi;
            cw = bm64[cwi];
            m = cw;
          }
          pw = cwi > 0 ? bm64[cwi - 1] : 0ull;
        }
        f = m ? (cwi << 6) + 63 - __builtin_clzll(m) : -1;  // -1: unreachable (w bits below f)
      }
    }
    if (lane < steps) E[xl] = el;
  }
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
    int32_t* __restrict__ ccnt, float* __restrict__ u_dmax) {
  __shared__ int s_c[kListWaves];
  // order codes of the largest delta per bucket: bucket i holds the keys of
  // tile t0+i's own rows, bucket 0 also every key before the group
  __shared__ uint32_t s_b[kSuperTiles];
  if (threadIdx.x < kSuperTiles) s_b[threadIdx.x] = 0u;  // 0: below every code
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
  if (lane == 0) atomicMax(&s_b[0], m0);
  __syncthreads();
  // tile t0+i: the largest delta over keys 0..p_hi, i.e. over buckets 0..i
  const int t0 = T * kSuperTiles;
  const int i = threadIdx.x;
  if (i < min(kSuperTiles, n_tiles - t0)) {
    uint32_t m = 0u;
    for (int k = 0; k <= i; ++k) m = max(m, s_b[k]);
    const uint32_t bits = (m & 0x80000000u) ? (m & 0x7fffffffu) : ~m;  // inverse of ord32
    u_dmax[(int64_t)seg * n_tiles + t0 + i] = __uint_as_float(bits);
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

// ---------------------------------------------------------------- decode: one row
// Keys 0..p of one sequence; keeps the w best (Hugging Face blog "Trainable
// Dynamic Mask Sparse Attention", section "Mask Combination with Causal
// Constraints": the top w of the causally visible keys by delta, ties to the
// lower index).  Thread t holds the codes of
// keys k*512 + t (coalesced loads, 64 registers).  The threshold, the largest
// code T with #{code >= T} >= w, is found bit by bit from the top.  The
// leading bits run over every key; the keys that can still reach the
// threshold (code >= the partial T, a few thousand for real rows) then move
// through LDS into 16 registers per thread for the remaining bits, unless
// there are more than kDecCand of them (ties), when the search stays on the
// full set.  The ordered output comes from two LDS bitmaps (code > T, and
// code == T for the ties, kept lowest index first), one 64-key tile per
// thread, which also gives the key-tile list.
constexpr int kDecThreads = 512;
constexpr int kDecWaves = kDecThreads / 64;
constexpr int kDecKPT = 64;          // rows up to 32768 keys
constexpr int kDecLead = 12;         // bits fixed over the full set
constexpr int kDecCand = 8192;       // candidates carried to the remaining bits
constexpr int kDecCPT = kDecCand / kDecThreads;

// Block total of per-thread counts in [0, 128): the wave sums its counts bit
// plane by bit plane with ballots (no cross-lane chains), one LDS slot per
// wave, one barrier.  Callers alternate two slot sets, which makes the one
// barrier enough: a wave cannot write a set again before every wave has
// passed the next call's barrier, i.e. finished reading it.
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

// One bit per round, hi down to lo: T | bit is taken when at least w codes
// reach it.  Padding codes are 0 and never reach a candidate (all >= 1).
// cge tracks #{code >= T}.
template <int K>
__device__ __forceinline__ uint32_t dec_bit_search(const uint32_t (&x)[K], uint32_t T, int hi,
                                                   int lo, int w, int* s_cnt, int& round,
                                                   int& cge) {
  for (int bit = hi; bit >= lo; --bit) {
    const uint32_t cand = T | (1u << bit);
    int c = 0;
#pragma unroll
    for (int k = 0; k < K; ++k) c += x[k] >= cand ? 1 : 0;
    const int tot = dec_block_count(c, s_cnt + (round & 1) * kDecWaves);
    ++round;
    if (tot >= w) {
      T = cand;
      cge = tot;
    }
  }
  return T;
}

template <int K>
__device__ __forceinline__ int dec_count_above(const uint32_t (&x)[K], uint32_t T, int* s_cnt,
                                               int& round) {
  int c = 0;
#pragma unroll
  for (int k = 0; k < K; ++k) c += x[k] > T ? 1 : 0;
  const int tot = dec_block_count(c, s_cnt + (round & 1) * kDecWaves);
  ++round;
  return tot;
}

__global__ __launch_bounds__(kDecThreads, 2) void decode_select_kernel(
    const float* __restrict__ delta, int Sk, int p, int w, int u_stride, int kt_stride,
    int32_t* __restrict__ u_idx, int32_t* __restrict__ u_cnt, int32_t* __restrict__ u_nfull,
    float* __restrict__ u_dmax, int32_t* __restrict__ kt_idx, int32_t* __restrict__ kt_cnt) {
  __shared__ int s_w[kDecWaves];
  __shared__ int s_cnt[2 * kDecWaves];
  __shared__ float s_m[kDecWaves];
  __shared__ __align__(8) uint32_t s_gt[kDecThreads * kDecKPT / 32];  // code > T (or all, n <= w)
  __shared__ __align__(8) uint32_t s_eq[kDecThreads * kDecKPT / 32];  // code == T
  __shared__ uint32_t s_cand[kDecCand];
  const int seg = blockIdx.x;
  const int n = p + 1;
  const float* Dl = delta + (int64_t)seg * Sk;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t code[kDecKPT];
  float mx = -INFINITY;
#pragma unroll
  for (int k = 0; k < kDecKPT; ++k) {
    const int j = k * kDecThreads + tid;
    const float v = Dl[min(j, n - 1)];  // every load issues before the first use
    code[k] = (j < n) ? dma::ord32(v) : 0u;
    mx = fmaxf(mx, v);  // the clamped key is a real one
  }
  mx = dma::wave_max(mx);
  if (lane == 0) s_m[wave] = mx;

  uint32_t T = 0;
  int need_eq = 0;
  if (n > w) {
    int round = 0, cge = n;
    T = dec_bit_search(code, T, 31, 32 - kDecLead, w, s_cnt, round, cge);
    int gt_tot;
    if (cge <= kDecCand) {
      // order-free compaction of the keys with code >= T
      int sc = 0;
#pragma unroll
      for (int k = 0; k < kDecKPT; ++k) sc += (k * kDecThreads + tid < n && code[k] >= T) ? 1 : 0;
      int stot;
      int at = block_excl_scan<kDecThreads>(sc, s_w, stot);
#pragma unroll
      for (int k = 0; k < kDecKPT; ++k)
        if (k * kDecThreads + tid < n && code[k] >= T && at < kDecCand) s_cand[at++] = code[k];
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
      T = dec_bit_search(code, T, 31 - kDecLead, 0, w, s_cnt, round, cge);
      gt_tot = dec_count_above(code, T, s_cnt, round);
    }
    need_eq = w - gt_tot;  // keys with code == T that are kept, lowest index first
  }
  // bitmaps of the verdicts: key k*512 + 64*wave + lane is bit lane of the
  // 64-bit word k*8 + wave
#pragma unroll
  for (int k = 0; k < kDecKPT; ++k) {
    const bool in = k * kDecThreads + tid < n;
    const uint64_t g = __ballot(in && (n <= w || code[k] > T));
    const uint64_t e = __ballot(in && n > w && code[k] == T);
    if (lane == 0) {
      reinterpret_cast<uint64_t*>(s_gt)[k * kDecWaves + wave] = g;
      reinterpret_cast<uint64_t*>(s_eq)[k * kDecWaves + wave] = e;
    }
  }
  __syncthreads();
  // thread t: keys [64t, 64t + 64), i.e. key tile t
  const uint64_t gt64 = reinterpret_cast<const uint64_t*>(s_gt)[tid];
  const uint64_t eq64 = reinterpret_cast<const uint64_t*>(s_eq)[tid];
  const int ne = __popcll(eq64);
  int etot;
  const int eb = block_excl_scan<kDecThreads>(ne, s_w, etot);
  const int allow = min(ne, max(0, need_eq - eb));
  uint64_t kept = gt64, x = eq64;
  for (int r = 0; r < allow; ++r) {
    kept |= x & (~x + 1ull);
    x &= x - 1ull;
  }
  const int nk = __popcll(kept);
  int tot;
  int pos = block_excl_scan<kDecThreads>(nk, s_w, tot);
  int32_t* out = u_idx + (int64_t)seg * u_stride;
  for (uint64_t y = kept; y; y &= y - 1ull) {
    if (pos < u_stride) out[pos] = 64 * tid + __builtin_ctzll(y);
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
    const int f = kept != 0ull ? 1 : 0;
    int ktot;
    const int at = block_excl_scan<kDecThreads>(f, s_w, ktot);
    if (f && at < kt_stride) kt_idx[(int64_t)seg * kt_stride + at] = tid;
    if (tid == 0) kt_cnt[seg] = min(ktot, kt_stride);
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
    int32_t* __restrict__ u_cnt, int32_t* __restrict__ u_nfull, float* __restrict__ u_dmax) {
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

// eviction checkpoints: every chk ranks, at most 64 per sequence
static int64_t ckpt_every(int64_t Sk) {
  const int64_t c = std::max<int64_t>(1024, (Sk + 63) / 64);
  return (c + 1023) & ~int64_t(1023);
}
static int64_t ckpt_words(int64_t Sk) { return (((Sk + 31) >> 5) + 3) & ~int64_t(3); }

size_t dma_topk_ws_bytes(int64_t BH, int64_t Sq, int64_t Sk, int64_t w) {
  // two key buffers (ping-pong merges), ranks, the candidate lists, then the
  // eviction checkpoints
  const size_t n = (size_t)BH * (size_t)Sk;
  const size_t ns = (size_t)BH * (size_t)n_super_of(Sq);
  const size_t nck = (size_t)BH * (size_t)((Sk + ckpt_every(Sk) - 1) / ckpt_every(Sk));
  return n * 2 * sizeof(uint64_t) + (size_t)BH * rank_stride(Sk) * sizeof(int32_t) +
         ns * (size_t)cand_cap(Sk, w) * 8 + ns * sizeof(int32_t) +
         nck * (size_t)ckpt_words(Sk) * sizeof(uint32_t) + 256;
}

hipError_t dma_launch_topk_prefill(const DmaTopkArgs& a, hipStream_t st) {
  const int64_t BH = a.B * a.Hkv;
  const int Sk = (int)a.Sk;
  const size_t n = (size_t)BH * (size_t)Sk;
  uint64_t* kA = static_cast<uint64_t*>(a.ws);
  uint64_t* kB = kA + n;
  int32_t* rank = reinterpret_cast<int32_t*>(kB + n);

  const int nch = (Sk + kSortChunk - 1) / kSortChunk;
  hipLaunchKernelGGL(sort_chunk_kernel, dim3(nch, BH), dim3(kSortThreads), 0, st, a.delta, Sk,
                     kA);
  uint64_t* src = kA;
  uint64_t* dst = kB;
  const int rs = (int)rank_stride(Sk);
  if (nch > 1 && nch <= kRankRunsMax) {
    const size_t lds = (size_t)Sk * sizeof(uint64_t);
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&rank_runs_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL(rank_runs_kernel, dim3(nch * (kSortChunk / kRankRunsKeys), BH),
                       dim3(kRankRunsThreads), lds, st, src, Sk, rs, rank, dst);
    src = dst;
  } else {
    for (int L = kSortChunk; L < Sk; L <<= 1) {
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
  if (n_chk > 1) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&ckpt_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)bm_bytes);
    hipLaunchKernelGGL(ckpt_kernel, dim3(n_chk - 1, BH), dim3(256), bm_bytes, st, rank, Sk, rs,
                       chk, n_chk, nwr, ckpt);
  }
  const int R = 64;
  const size_t ev_lds = bm_bytes + 8 * sizeof(int);  // bitmap, then s_w[4], s_f (padded)
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&evict_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)ev_lds);
  hipLaunchKernelGGL(evict_kernel, dim3((Sk + R - 1) / R, BH), dim3(256), ev_lds, st, src, Sk,
                     (int)a.w, R, chk, n_chk, nwr, ckpt, a.evict);
  hipLaunchKernelGGL(cand_kernel, dim3(n_super, BH), dim3(kListWaves * 64), 0, st, a.delta,
                     a.evict, Sk, (int)a.Sq, (int)a.q0, n_super, (int)a.n_tiles, cap, cj, ce, ccnt,
                     a.u_dmax);
  const size_t kt_lds =
      a.kt_idx ? (size_t)kSuperTiles * ((a.kt_stride + 31) / 32) * sizeof(uint32_t) : 0;
  if (kt_lds > (size_t)kSuperTiles * kMaxKtWords * sizeof(uint32_t)) return hipErrorInvalidValue;
  if (kt_lds > 0)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&group_lists_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)kt_lds);
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
                     tile_dmax);
  return hipGetLastError();
}

hipError_t dma_launch_decode_append(const float* delta, int64_t BH, int64_t Sk, int64_t w,
                                   int32_t* u_idx, int32_t* u_cnt, int32_t* u_nfull,
                                   float* u_dmax, hipStream_t st) {
  const size_t lds = (size_t)w * sizeof(int32_t);
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_append_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  hipLaunchKernelGGL(decode_append_kernel, dim3((unsigned)BH), dim3(kAppThreads), lds, st, delta,
                     (int)Sk, (int)w, u_idx, u_cnt, u_nfull, u_dmax);
  return hipGetLastError();
}

hipError_t dma_launch_topk_decode(const DmaTopkArgs& a, hipStream_t st) {
  const int64_t BH = a.B * a.Hkv;
  hipLaunchKernelGGL(decode_select_kernel, dim3(BH), dim3(kDecThreads), 0, st, a.delta, (int)a.Sk,
                     (int)a.q0, (int)a.w, (int)a.u_stride, (int)a.kt_stride, a.u_idx, a.u_cnt,
                     a.u_nfull, a.u_dmax, a.kt_idx, a.kt_cnt);
  return hipGetLastError();
}
