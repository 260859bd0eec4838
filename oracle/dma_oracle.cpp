// fp64 CPU oracle for the Dynamic Mask Attention (DMA) forward and backward.
//
// TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
// baseline leg of the benchmark may load this library.  It shares no code,
// header, table or helper with the HIP path under trainable_dynamic_mask_amd/.
//
// Every quantity is computed in double precision, the plain way, straight
// from the definitions on the Hugging Face blog "Trainable Dynamic Mask
// Sparse Attention" (cited below as "the DMA blog"):
//   * dynamic weights   delta = exp(tau(v Delta) x A)      (section "Dynamic
//     Sparse Mask Generation", the delta equation), tau = softplus;
//   * keep mask         m_t = f(top_w(delta + m_c^t))       (section "Mask
//     Combination with Causal Constraints"): among the causally valid keys
//     j <= p of query position p keep the w largest delta, ties broken toward
//     the lower key index; f writes -inf everywhere else;
//   * attention         o_t = softmax(q_t k^T / sqrt(d_h) o m_t) v  (section
//     "Efficient Sparse Attention Computation"), with "o" read as adding m_t
//     (delta on kept keys, -inf elsewhere) to the scaled scores.
// The keep set of each query row is found by direct selection over that
// row's candidates (std::nth_element), never through any property of the
// rows' sets, so the oracle stays independent of how the GPU builds masks.
//
// Inputs: Q, K, V are float32 arrays holding the exact values the GPU sees
// (bf16 values widen to float32 without rounding); Delta and A are float32.
// Layouts: Q [B, Sq, Hq, D], K and V [B, Sk, Hkv, D], Delta [Hkv*D, Hkv],
// A [Hkv], delta [B, Hkv, Sk]; all row-major and contiguous.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <numeric>
#include <vector>
#include <omp.h>

namespace {

// softplus(x) = log(1 + e^x) evaluated without overflow.
double softplus(double x) {
  return x > 0.0 ? x + std::log1p(std::exp(-x)) : std::log1p(std::exp(x));
}

// Key a beats key b: larger delta, or equal delta and lower index.
struct Beats {
  const double* d;
  bool operator()(int32_t a, int32_t b) const {
    return d[a] > d[b] || (d[a] == d[b] && a < b);
  }
};

// Keep set of query position p over keys 0..p, ascending.  Returns its size.
int64_t keep_row(const double* d, int64_t p, int64_t w, int32_t* out,
                 std::vector<int32_t>& scratch) {
  const int64_t n = p + 1;
  if (n <= w) {
    for (int64_t j = 0; j < n; ++j) out[j] = (int32_t)j;
    return n;
  }
  scratch.resize(n);
  std::iota(scratch.begin(), scratch.end(), 0);
  Beats beats{d};
  std::nth_element(scratch.begin(), scratch.begin() + (w - 1), scratch.end(), beats);
  const int32_t t = scratch[w - 1];  // the w-th best candidate
  int64_t c = 0;
  for (int64_t j = 0; j < n; ++j)
    if (!beats(t, (int32_t)j)) out[c++] = (int32_t)j;  // j == t or j beats t
  return c;
}

}  // namespace

extern "C" {

int orc_num_threads() { return omp_get_max_threads(); }

// Dynamic weights (DMA blog, delta equation):
//   pre[b,j,h] = sum_c V[b,j,c] * Delta[c,h], c = kv_head*D + channel
//   delta[b,h,j] = exp(softplus(pre) * A[h])
void orc_weights(const float* V, const float* Delta, const float* A, int64_t B, int64_t Sk,
                 int64_t Hkv, int64_t D, double* delta) {
  const int64_t C = Hkv * D;
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t b = 0; b < B; ++b)
    for (int64_t j = 0; j < Sk; ++j) {
      const float* v = V + (b * Sk + j) * C;
      for (int64_t h = 0; h < Hkv; ++h) {
        double pre = 0.0;
        for (int64_t c = 0; c < C; ++c) pre += (double)v[c] * (double)Delta[c * Hkv + h];
        delta[(b * Hkv + h) * Sk + j] = std::exp(softplus(pre) * (double)A[h]);
      }
    }
}

// Value projection, the linear map whose output is the value matrix the
// delta equation starts from (DMA blog, section "Dynamic Sparse Mask
// Generation"):  V[m, n] = sum_k X[m, k] * Wv[k, n]  over the M = B*Sk rows,
// each sum taken in order of k.
void orc_vproj(const float* X, const float* Wv, int64_t M, int64_t Cin, int64_t N, double* V) {
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; ++m) {
    double* out = V + m * N;
    for (int64_t n = 0; n < N; ++n) out[n] = 0.0;
    for (int64_t k = 0; k < Cin; ++k) {
      const double x = (double)X[m * Cin + k];
      const float* wrow = Wv + k * N;
      for (int64_t n = 0; n < N; ++n) out[n] += x * (double)wrow[n];
    }
  }
}

// Keep set of one query position p (keys 0..p of one delta row), ascending.
int64_t orc_keep_row(const double* d, int64_t p, int64_t w, int32_t* out) {
  std::vector<int32_t> scratch;
  return keep_row(d, p, w, out, scratch);
}

// Mask over query positions [q0, q0+Sq) of BH independent delta rows of
// length Sk, built from the literal per-row keep sets.
//   evict[bh, j]: one past the last observed row that keeps key j; when no
//     observed row keeps j it is max(j, q0).  Before writing it, checks that
//     the observed rows keeping j form
//     the contiguous run [max(j,q0), evict) and returns -1 (after finishing)
//     if any key breaks that.
//   Tiles of Bq consecutive rows (tile t covers rows q0+t*Bq ...):
//     u_cnt[bh, t] keys kept by at least one row of the tile, listed
//     ascending at u_idx[(bh*nQT + t)*u_stride ...];
//     kt_cnt[bh, t] key tiles [kt*Bk, (kt+1)*Bk) holding at least one such
//     key, listed ascending at kt_idx[(bh*nQT + t)*kt_stride ...].
//   row_cnt[bh, r] size of the keep set of row q0+r.
// Returns 0, -1 (interval check failed) or -2 (a list overflowed its stride).
int orc_mask(const double* delta, int64_t BH, int64_t Sk, int64_t q0, int64_t Sq, int64_t w,
             int64_t Bq, int64_t Bk, int32_t* evict, int64_t* row_cnt, int64_t* u_cnt,
             int32_t* u_idx, int64_t u_stride, int64_t* kt_cnt, int32_t* kt_idx,
             int64_t kt_stride) {
  const int64_t nQT = (Sq + Bq - 1) / Bq;
  const int64_t nKT = (Sk + Bk - 1) / Bk;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
  for (int64_t bh = 0; bh < BH; ++bh) {
    const double* d = delta + bh * Sk;
    std::vector<int32_t> scratch, row(Sk > 0 ? Sk : 1);
    std::vector<int64_t> first(Sk, -1), last(Sk, -1), cnt(Sk, 0);
    std::vector<char> in_tile(Sk, 0), kt_on(nKT > 0 ? nKT : 1, 0);
    for (int64_t t = 0; t < nQT; ++t) {
      std::fill(in_tile.begin(), in_tile.end(), 0);
      const int64_t r0 = t * Bq, r1 = std::min(Sq, r0 + Bq);
      for (int64_t r = r0; r < r1; ++r) {
        const int64_t p = q0 + r;
        const int64_t n = keep_row(d, p, w, row.data(), scratch);
        row_cnt[bh * Sq + r] = n;
        for (int64_t k = 0; k < n; ++k) {
          const int32_t j = row[k];
          if (first[j] < 0) first[j] = p;
          last[j] = p;
          cnt[j] += 1;
          in_tile[j] = 1;
        }
      }
      // tile lists, ascending
      int64_t nu = 0;
      std::fill(kt_on.begin(), kt_on.end(), 0);
      int32_t* ul = u_idx + (bh * nQT + t) * u_stride;
      for (int64_t j = 0; j < Sk; ++j)
        if (in_tile[j]) {
          if (nu < u_stride) ul[nu] = (int32_t)j; else bad |= 2;
          ++nu;
          kt_on[j / Bk] = 1;
        }
      u_cnt[bh * nQT + t] = nu;
      int64_t nk = 0;
      int32_t* kl = kt_idx + (bh * nQT + t) * kt_stride;
      for (int64_t kt = 0; kt < nKT; ++kt)
        if (kt_on[kt]) {
          if (nk < kt_stride) kl[nk] = (int32_t)kt; else bad |= 2;
          ++nk;
        }
      kt_cnt[bh * nQT + t] = nk;
    }
    for (int64_t j = 0; j < Sk; ++j) {
      const int64_t start = std::max<int64_t>(j, q0);
      if (cnt[j] > 0 && (first[j] != start || last[j] - first[j] + 1 != cnt[j])) bad |= 1;
      evict[bh * Sk + j] = (int32_t)(cnt[j] > 0 ? last[j] + 1 : start);
    }
  }
  if (bad & 2) return -2;
  if (bad & 1) return -1;
  return 0;
}

// Attention for a list of query rows (DMA blog, attention equation with
// the additive reading of the mask):
//   for row (b, hq, i) at position p = q0 + i with kv head h = hq / (Hq/Hkv):
//   s_j = scale * (q . k_j) + delta[b,h,j] for j in keep(p)
//   o   = sum_j exp(s_j - m) v_j / sum_j exp(s_j - m),  m = max_j s_j
//   lse = m + log(sum_j exp(s_j - m))
// rows: n triples (b, hq, i).  O: [n, D]; lse: [n].
void orc_attn_rows(const float* Q, const float* K, const float* V, const double* delta,
                   int64_t B, int64_t Sq, int64_t Sk, int64_t Hq, int64_t Hkv, int64_t D,
                   int64_t q0, int64_t w, double scale, const int64_t* rows, int64_t n,
                   double* O, double* lse) {
  (void)B;
  const int64_t G = Hq / Hkv;
#pragma omp parallel
  {
    std::vector<int32_t> scratch, keep(Sk > 0 ? Sk : 1);
    std::vector<double> s(Sk > 0 ? Sk : 1), acc(D);
#pragma omp for schedule(dynamic, 4)
    for (int64_t r = 0; r < n; ++r) {
      const int64_t b = rows[3 * r], hq = rows[3 * r + 1], i = rows[3 * r + 2];
      const int64_t h = hq / G, p = q0 + i;
      const double* d = delta + (b * Hkv + h) * Sk;
      const int64_t nk = keep_row(d, p, w, keep.data(), scratch);
      const float* q = Q + ((b * Sq + i) * Hq + hq) * D;
      double m = -INFINITY;
      for (int64_t k = 0; k < nk; ++k) {
        const int64_t j = keep[k];
        const float* kr = K + ((b * Sk + j) * Hkv + h) * D;
        double dot = 0.0;
        for (int64_t c = 0; c < D; ++c) dot += (double)q[c] * (double)kr[c];
        s[k] = scale * dot + d[j];
        m = std::max(m, s[k]);
      }
      double z = 0.0;
      std::fill(acc.begin(), acc.end(), 0.0);
      for (int64_t k = 0; k < nk; ++k) {
        const int64_t j = keep[k];
        const double e = std::exp(s[k] - m);
        z += e;
        const float* vr = V + ((b * Sk + j) * Hkv + h) * D;
        for (int64_t c = 0; c < D; ++c) acc[c] += e * (double)vr[c];
      }
      for (int64_t c = 0; c < D; ++c) O[r * D + c] = acc[c] / z;
      lse[r] = m + std::log(z);
    }
  }
}

// Backward of the attention (gradient of L = sum over rows of dO . O, the
// keep sets held fixed: they are piecewise constant in delta).  For row
// (b, hq, i) at position p = q0 + i over its kept keys J, with
// P_j = exp(s_j - lse) and O = sum_j P_j v_j as in orc_attn_rows:
//   Dr   = dO . O
//   dP_j = dO . v_j,   dS_j = P_j (dP_j - Dr)       (softmax Jacobian)
//   dQ_i = scale sum_j dS_j k_j
//   dK_j += scale dS_j q_i,   dV_j += P_j dO,   ddelta[b,h,j] += dS_j
// Every (batch, kv head) sequence owns its dK/dV/ddelta rows, so sequences run
// in parallel and each walks its G query heads and Sq rows in order.
// Layouts as orc_attn_rows; dO [B,Sq,Hq,D]; dQ [B,Sq,Hq,D]; dK, dV
// [B,Sk,Hkv,D]; ddelta [B,Hkv,Sk]; all outputs are overwritten.
void orc_attn_bwd(const float* Q, const float* K, const float* V, const double* delta,
                  const float* dO, int64_t B, int64_t Sq, int64_t Sk, int64_t Hq, int64_t Hkv,
                  int64_t D, int64_t q0, int64_t w, double scale, double* dQ, double* dK,
                  double* dV, double* ddelta) {
  const int64_t G = Hq / Hkv;
  std::fill(dK, dK + B * Sk * Hkv * D, 0.0);
  std::fill(dV, dV + B * Sk * Hkv * D, 0.0);
  std::fill(ddelta, ddelta + B * Hkv * Sk, 0.0);
#pragma omp parallel
  {
    std::vector<int32_t> scratch, keep(Sk > 0 ? Sk : 1);
    std::vector<double> s(Sk > 0 ? Sk : 1), P(Sk > 0 ? Sk : 1), o(D), dq(D);
#pragma omp for collapse(2) schedule(dynamic, 1)
    for (int64_t b = 0; b < B; ++b)
      for (int64_t h = 0; h < Hkv; ++h) {
        const double* d = delta + (b * Hkv + h) * Sk;
        for (int64_t hq = h * G; hq < (h + 1) * G; ++hq)
          for (int64_t i = 0; i < Sq; ++i) {
            const int64_t p = q0 + i;
            const int64_t nk = keep_row(d, p, w, keep.data(), scratch);
            const float* q = Q + ((b * Sq + i) * Hq + hq) * D;
            const float* g = dO + ((b * Sq + i) * Hq + hq) * D;
            double m = -INFINITY;
            for (int64_t k = 0; k < nk; ++k) {
              const float* kr = K + ((b * Sk + keep[k]) * Hkv + h) * D;
              double dot = 0.0;
              for (int64_t c = 0; c < D; ++c) dot += (double)q[c] * (double)kr[c];
              s[k] = scale * dot + d[keep[k]];
              m = std::max(m, s[k]);
            }
            double z = 0.0;
            for (int64_t k = 0; k < nk; ++k) z += std::exp(s[k] - m);
            const double lse = m + std::log(z);
            std::fill(o.begin(), o.end(), 0.0);
            for (int64_t k = 0; k < nk; ++k) {
              P[k] = std::exp(s[k] - lse);
              const float* vr = V + ((b * Sk + keep[k]) * Hkv + h) * D;
              for (int64_t c = 0; c < D; ++c) o[c] += P[k] * (double)vr[c];
            }
            double Dr = 0.0;
            for (int64_t c = 0; c < D; ++c) Dr += (double)g[c] * o[c];
            std::fill(dq.begin(), dq.end(), 0.0);
            for (int64_t k = 0; k < nk; ++k) {
              const int64_t j = keep[k];
              const float* kr = K + ((b * Sk + j) * Hkv + h) * D;
              const float* vr = V + ((b * Sk + j) * Hkv + h) * D;
              double dp = 0.0;
              for (int64_t c = 0; c < D; ++c) dp += (double)g[c] * (double)vr[c];
              const double ds = P[k] * (dp - Dr);
              double* dk = dK + ((b * Sk + j) * Hkv + h) * D;
              double* dv = dV + ((b * Sk + j) * Hkv + h) * D;
              for (int64_t c = 0; c < D; ++c) {
                dq[c] += ds * (double)kr[c];
                dk[c] += scale * ds * (double)q[c];
                dv[c] += P[k] * (double)g[c];
              }
              ddelta[(b * Hkv + h) * Sk + j] += ds;
            }
            double* dqo = dQ + ((b * Sq + i) * Hq + hq) * D;
            for (int64_t c = 0; c < D; ++c) dqo[c] = scale * dq[c];
          }
      }
  }
}

// The same backward for sampled outputs, for sizes where the whole backward
// is too slow.  orc_attn_bwd_rows: dQ of the listed (b, hq, i) rows (a row's
// dQ depends on that row only).  orc_attn_bwd_keys: dK, dV and ddelta of the
// listed (b, h, j) keys, summing over every row p >= j whose keep set holds
// j, for each of the G query heads of kv head h.  dQ [n, D]; dK, dV [m, D];
// ddelta [m].
namespace {
// P, s and the keep set of row (b, hq, i); returns its size; fills O.
int64_t row_probs(const float* Q, const float* K, const float* V, const double* d, int64_t b,
                  int64_t hq, int64_t i, int64_t h, int64_t Sq, int64_t Sk, int64_t Hq,
                  int64_t Hkv, int64_t D, int64_t q0, int64_t w, double scale,
                  std::vector<int32_t>& keep, std::vector<int32_t>& scratch,
                  std::vector<double>& s, std::vector<double>& P, std::vector<double>& o) {
  const int64_t nk = keep_row(d, q0 + i, w, keep.data(), scratch);
  const float* q = Q + ((b * Sq + i) * Hq + hq) * D;
  double m = -INFINITY;
  for (int64_t k = 0; k < nk; ++k) {
    const float* kr = K + ((b * Sk + keep[k]) * Hkv + h) * D;
    double dot = 0.0;
    for (int64_t c = 0; c < D; ++c) dot += (double)q[c] * (double)kr[c];
    s[k] = scale * dot + d[keep[k]];
    m = std::max(m, s[k]);
  }
  double z = 0.0;
  for (int64_t k = 0; k < nk; ++k) z += std::exp(s[k] - m);
  const double lse = m + std::log(z);
  std::fill(o.begin(), o.end(), 0.0);
  for (int64_t k = 0; k < nk; ++k) {
    P[k] = std::exp(s[k] - lse);
    const float* vr = V + ((b * Sk + keep[k]) * Hkv + h) * D;
    for (int64_t c = 0; c < D; ++c) o[c] += P[k] * (double)vr[c];
  }
  return nk;
}
}  // namespace

void orc_attn_bwd_rows(const float* Q, const float* K, const float* V, const double* delta,
                       const float* dO, int64_t Sq, int64_t Sk, int64_t Hq, int64_t Hkv,
                       int64_t D, int64_t q0, int64_t w, double scale, const int64_t* rows,
                       int64_t n, double* dQ) {
  const int64_t G = Hq / Hkv;
#pragma omp parallel
  {
    std::vector<int32_t> scratch, keep(Sk > 0 ? Sk : 1);
    std::vector<double> s(Sk > 0 ? Sk : 1), P(Sk > 0 ? Sk : 1), o(D);
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < n; ++r) {
      const int64_t b = rows[3 * r], hq = rows[3 * r + 1], i = rows[3 * r + 2], h = hq / G;
      const double* d = delta + (b * Hkv + h) * Sk;
      const int64_t nk = row_probs(Q, K, V, d, b, hq, i, h, Sq, Sk, Hq, Hkv, D, q0, w, scale,
                                   keep, scratch, s, P, o);
      const float* g = dO + ((b * Sq + i) * Hq + hq) * D;
      double Dr = 0.0;
      for (int64_t c = 0; c < D; ++c) Dr += (double)g[c] * o[c];
      double* out = dQ + r * D;
      std::fill(out, out + D, 0.0);
      for (int64_t k = 0; k < nk; ++k) {
        const float* kr = K + ((b * Sk + keep[k]) * Hkv + h) * D;
        const float* vr = V + ((b * Sk + keep[k]) * Hkv + h) * D;
        double dp = 0.0;
        for (int64_t c = 0; c < D; ++c) dp += (double)g[c] * (double)vr[c];
        const double ds = P[k] * (dp - Dr);
        for (int64_t c = 0; c < D; ++c) out[c] += scale * ds * (double)kr[c];
      }
    }
  }
}

void orc_attn_bwd_keys(const float* Q, const float* K, const float* V, const double* delta,
                       const float* dO, int64_t Sq, int64_t Sk, int64_t Hq, int64_t Hkv,
                       int64_t D, int64_t q0, int64_t w, double scale, const int64_t* keys,
                       int64_t m, double* dK, double* dV, double* ddelta) {
  const int64_t G = Hq / Hkv;
  for (int64_t t = 0; t < m; ++t) {
    const int64_t b = keys[3 * t], h = keys[3 * t + 1], j = keys[3 * t + 2];
    const double* d = delta + (b * Hkv + h) * Sk;
    std::vector<double> gk(D, 0.0), gv(D, 0.0);
    double gd = 0.0;
#pragma omp parallel
    {
      std::vector<int32_t> scratch, keep(Sk > 0 ? Sk : 1);
      std::vector<double> s(Sk > 0 ? Sk : 1), P(Sk > 0 ? Sk : 1), o(D), lk(D, 0.0), lv(D, 0.0);
      double ld = 0.0;
#pragma omp for collapse(2) schedule(dynamic, 4)
      for (int64_t hq = h * G; hq < (h + 1) * G; ++hq)
        for (int64_t i = std::max<int64_t>(0, j - q0); i < Sq; ++i) {
          const int64_t nk = row_probs(Q, K, V, d, b, hq, i, h, Sq, Sk, Hq, Hkv, D, q0, w, scale,
                                       keep, scratch, s, P, o);
          int64_t kj = -1;
          for (int64_t k = 0; k < nk; ++k)
            if (keep[k] == j) kj = k;
          if (kj < 0) continue;
          const float* g = dO + ((b * Sq + i) * Hq + hq) * D;
          const float* q = Q + ((b * Sq + i) * Hq + hq) * D;
          const float* vr = V + ((b * Sk + j) * Hkv + h) * D;
          double Dr = 0.0, dp = 0.0;
          for (int64_t c = 0; c < D; ++c) {
            Dr += (double)g[c] * o[c];
            dp += (double)g[c] * (double)vr[c];
          }
          const double ds = P[kj] * (dp - Dr);
          for (int64_t c = 0; c < D; ++c) {
            lk[c] += scale * ds * (double)q[c];
            lv[c] += P[kj] * (double)g[c];
          }
          ld += ds;
        }
#pragma omp critical
      {
        for (int64_t c = 0; c < D; ++c) {
          gk[c] += lk[c];
          gv[c] += lv[c];
        }
        gd += ld;
      }
    }
    for (int64_t c = 0; c < D; ++c) {
      dK[t * D + c] = gk[c];
      dV[t * D + c] = gv[c];
    }
    ddelta[t] = gd;
  }
}

// Backward of the dynamic weights, given ddelta = dL/ddelta:
//   pre = sum_c V[b,j,c] Delta[c,h],  sp = softplus(pre),  delta = exp(sp A[h])
//   dpre = ddelta * delta * A[h] * sigmoid(pre)      (softplus' = sigmoid)
//   dA[h]       += ddelta * delta * sp
//   dDelta[c,h] += V[b,j,c] * dpre
//   dV[b,j,c]    = sum_h dpre[h] * Delta[c,h]
// dV [B,Sk,Hkv*D] (overwritten; add the attention's dV separately),
// dDelta [Hkv*D, Hkv], dA [Hkv] (overwritten).
void orc_weights_bwd(const float* V, const float* Delta, const float* A, const double* ddelta,
                     int64_t B, int64_t Sk, int64_t Hkv, int64_t D, double* dV, double* dDelta,
                     double* dA) {
  const int64_t C = Hkv * D;
  std::fill(dDelta, dDelta + C * Hkv, 0.0);
  std::fill(dA, dA + Hkv, 0.0);
#pragma omp parallel
  {
    std::vector<double> gD(C * Hkv, 0.0), gA(Hkv, 0.0), dpre(Hkv);
#pragma omp for collapse(2) schedule(static)
    for (int64_t b = 0; b < B; ++b)
      for (int64_t j = 0; j < Sk; ++j) {
        const float* v = V + (b * Sk + j) * C;
        for (int64_t h = 0; h < Hkv; ++h) {
          double pre = 0.0;
          for (int64_t c = 0; c < C; ++c) pre += (double)v[c] * (double)Delta[c * Hkv + h];
          const double sp = softplus(pre);
          const double dl = std::exp(sp * (double)A[h]);
          const double gd = ddelta[(b * Hkv + h) * Sk + j];
          const double sig = 1.0 / (1.0 + std::exp(-pre));
          dpre[h] = gd * dl * (double)A[h] * sig;
          gA[h] += gd * dl * sp;
          for (int64_t c = 0; c < C; ++c) gD[c * Hkv + h] += (double)v[c] * dpre[h];
        }
        double* dv = dV + (b * Sk + j) * C;
        for (int64_t c = 0; c < C; ++c) {
          double acc = 0.0;
          for (int64_t h = 0; h < Hkv; ++h) acc += dpre[h] * (double)Delta[c * Hkv + h];
          dv[c] = acc;
        }
      }
#pragma omp critical
    {
      for (int64_t k = 0; k < C * Hkv; ++k) dDelta[k] += gD[k];
      for (int64_t h = 0; h < Hkv; ++h) dA[h] += gA[h];
    }
  }
}

}  // extern "C"
