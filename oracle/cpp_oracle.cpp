// Plain fp64 CPU oracle of exact attention -- TEST INFRASTRUCTURE ONLY.
//
// This file is the reference the GPU kernels are checked against.  It is
// written to be read against the pages, not to be fast: every score matrix S
// and probability matrix P is materialised (one panel of rows at a time), the
// softmax takes two passes over each row (the max, then the exponentials and
// their sum), and every product is a plain loop.  Only the tests, the smoke
// check and the CPU-baseline leg of the benchmark load it; the library and its
// binding never do, and this file includes nothing of theirs.
//
// Definitions followed:
//  * attention: S = scale * Q K^T, P = softmax(S) row by row, O = P V -- the
//    standard-attention formula of the FlashAttention (TH) page (section on
//    standard attention) and the ledger page ("FLOPs" section); LSE = m + ln l
//    with m the row max and l the sum of exponentials that the online softmax
//    keeps (FlashAttention (TH) page, online softmax; natural log).
//  * causal: row i sees keys j <= i (the lower-triangular mask of the HSTU
//    page, optimisation two, read with the diagonal kept).
//  * grouped-query attention: query head h reads key/value head h / (H/Hkv).
//  * decode: one query per sequence against cache rows [0, L_b) (ledger page,
//    bandwidth section: s_j = q.k_j over the history, o = sum_j p_j v_j).
//  * paged decode: logical key j of sequence b is row j % P of physical page
//    table[b][j / P] (the PagedAttention scheme that the CANN ops-transformer
//    FlashAttention page names under KV-cache management).
//  * HSTU: x = Q K^T; x *= alpha; x = silu(x); x *= mask / n; O = x V, in the
//    order of the HSTU page's listing, per packed sequence (optimisation
//    three: jagged tensors, no cross-sequence terms).
//  * backward: the chain rule of the forward definition, dV = P^T dO,
//    dP = dO V^T, D_i = sum_j P_ij dP_ij, dS = P * (dP - D), dQ = scale dS K,
//    dK = scale dS^T Q (the ledger page names the backward pass by its n x n
//    intermediates in its memory section).
//
// Loop order: every product is written as a loop over the contraction index
// outside a loop over output columns (an "axpy" of one row), so that each
// output element is summed in the order of its contraction index, exactly as
// the sum is written, while the inner loop runs over contiguous memory.
//
// Work is split over OpenMP threads by (batch, head, row panel) -- units that
// share nothing -- so each output element is written by exactly one thread
// and the results do not depend on the thread count.
//
// Every product loop adds its length to a multiply-add counter, so that the
// FLOP convention (two products of n^2 d multiply-adds per head) can be
// checked against what the loops actually executed.
#include <omp.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <vector>

namespace {

constexpr double kNegInf = -std::numeric_limits<double>::infinity();

// Rows per materialised panel: the whole query range for short key ranges
// (tiny self-tests see all of S and P), otherwise 2^20 / Nk rows, so S and P
// stay at 8 MB each per thread whatever the sequence length.  Rows are
// independent under the definition, so panels change nothing in the result.
int64_t panel_rows(int64_t nrows, int64_t nk) {
  if (nk <= 1024) return std::max<int64_t>(1, nrows);
  return std::max<int64_t>(1, (int64_t(1) << 20) / nk);
}

// Keys visible from query row i among nk keys: a prefix [0, nvis).
int64_t visible(int64_t i, int64_t nk, int causal) { return causal ? std::min(i + 1, nk) : nk; }

// y[0..n) += a * x[0..n)
__attribute__((target_clones("arch=haswell", "default"))) void axpy(double a, const double* x, double* y,
                                                                      int64_t n) {
  for (int64_t t = 0; t < n; ++t) y[t] += a * x[t];
}

// Scores of one query row against the first nvis keys:
// s[j] = scale * sum_c q[c] * kt[c][j], with kt = K^T ([d][ldk]).
void score_row(const double* q, const double* kt, int64_t ldk, int64_t d, int64_t nvis, double scale, double* s,
               int64_t& macs) {
  std::fill(s, s + nvis, 0.0);
  for (int64_t c = 0; c < d; ++c) {
    axpy(q[c], kt + c * ldk, s, nvis);
    macs += nvis;
  }
  for (int64_t j = 0; j < nvis; ++j) s[j] *= scale;
}

// Two-pass softmax of one materialised score row s[0..nvis) (the masked
// entries are not stored): pass 1 the max m, pass 2 p = exp(s - m) and their
// sum l; then p /= l.  A row with no visible key gets p = 0, m = -inf, l = 0.
void softmax_row(const double* s, double* p, int64_t nvis, double& m, double& l) {
  m = kNegInf;
  for (int64_t j = 0; j < nvis; ++j) m = std::max(m, s[j]);
  l = 0.0;
  if (nvis == 0 || m == kNegInf) {
    std::fill(p, p + nvis, 0.0);
    return;
  }
  for (int64_t j = 0; j < nvis; ++j) {
    p[j] = std::exp(s[j] - m);
    l += p[j];
  }
  for (int64_t j = 0; j < nvis; ++j) p[j] /= l;
}

// o[0..dv) = sum_{j < nvis} p[j] * v[j][0..dv)
void pv_row(const double* p, const double* v, int64_t ldv, int64_t dv, int64_t nvis, double* o, int64_t& macs) {
  std::fill(o, o + dv, 0.0);
  for (int64_t j = 0; j < nvis; ++j) {
    axpy(p[j], v + j * ldv, o, dv);
    macs += dv;
  }
}

// K^T of one head: kt[c][j] = k[j][c], c < d, j < nk.
void transpose(const double* k, int64_t nk, int64_t d, double* kt) {
  for (int64_t j = 0; j < nk; ++j)
    for (int64_t c = 0; c < d; ++c) kt[c * nk + j] = k[j * d + c];
}

}  // namespace

extern "C" {

int oracle_max_threads(void) { return omp_get_max_threads(); }
void oracle_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }

// Exact attention forward.
//   q [B,H,Nq,d], k [B,Hkv,Nk,d], v [B,Hkv,Nk,dv]; rows [nrows] (query rows to
//   compute, in [0, Nq)), or null for all rows (nrows = Nq).
//   o [B,H,nrows,dv], lse [B,H,nrows] written; probs [B,H,nrows,Nk] written if
//   non-null (the materialised P, zeros where masked).
//   macs (optional) receives the multiply-adds executed in the two products.
void oracle_attention_forward(const double* q, const double* k, const double* v, int64_t B, int64_t H, int64_t Hkv,
                              int64_t Nq, int64_t Nk, int64_t d, int64_t dv, double scale, int causal,
                              const int64_t* rows, int64_t nrows, double* o, double* lse, double* probs,
                              int64_t* macs) {
  if (!rows) nrows = Nq;
  const int64_t group = H / Hkv;
  const int64_t R = panel_rows(nrows, Nk);
  const int64_t npanel = (nrows + R - 1) / R;
  const int64_t ntask = B * H * npanel;
  int64_t total = 0;
#pragma omp parallel reduction(+ : total)
  {
    std::vector<double> kt((size_t)d * Nk), S((size_t)R * Nk), P((size_t)R * Nk);
    int64_t kt_head = -1;
#pragma omp for schedule(dynamic, 1)
    for (int64_t t = 0; t < ntask; ++t) {
      const int64_t p0 = (t % npanel) * R;
      const int64_t bh = t / npanel;
      const int64_t b = bh / H, h = bh % H, g = h / group;
      const int64_t kvh = b * Hkv + g;
      const double* kh = k + kvh * Nk * d;
      const double* vh = v + kvh * Nk * dv;
      if (kt_head != kvh) {
        transpose(kh, Nk, d, kt.data());
        kt_head = kvh;
      }
      const int64_t pr = std::min(R, nrows - p0);
      // 1. S of the panel (masked entries -inf), 2. P by a two-pass softmax
      for (int64_t r = 0; r < pr; ++r) {
        const int64_t i = rows ? rows[p0 + r] : p0 + r;
        const int64_t nv = visible(i, Nk, causal);
        double* s = S.data() + r * Nk;
        double* p = P.data() + r * Nk;
        score_row(q + (bh * Nq + i) * d, kt.data(), Nk, d, nv, scale, s, total);
        std::fill(s + nv, s + Nk, kNegInf);
        double m, l;
        softmax_row(s, p, nv, m, l);
        std::fill(p + nv, p + Nk, 0.0);
        lse[bh * nrows + p0 + r] = (l > 0.0) ? m + std::log(l) : kNegInf;
      }
      // 3. O = P V
      for (int64_t r = 0; r < pr; ++r) {
        const int64_t i = rows ? rows[p0 + r] : p0 + r;
        pv_row(P.data() + r * Nk, vh, dv, dv, visible(i, Nk, causal), o + (bh * nrows + p0 + r) * dv, total);
        if (probs) std::memcpy(probs + (bh * nrows + p0 + r) * Nk, P.data() + r * Nk, sizeof(double) * Nk);
      }
    }
  }
  if (macs) *macs = total;
}

// Decode: q [B,H,d] against caches [B,Hkv,Lmax,d] (v: dv columns), row b
// attending to cache rows [0, seqlens[b]).  o [B,H,dv], lse [B,H].  A sequence
// with no row gets O = 0 and LSE = -inf.
void oracle_decode(const double* q, const double* kc, const double* vc, const int64_t* seqlens, int64_t B, int64_t H,
                   int64_t Hkv, int64_t Lmax, int64_t d, int64_t dv, double scale, double* o, double* lse,
                   int64_t* macs) {
  const int64_t group = H / Hkv;
  int64_t total = 0;
#pragma omp parallel reduction(+ : total)
  {
    std::vector<double> kt, S, P;
#pragma omp for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < B * H; ++bh) {
      const int64_t b = bh / H, h = bh % H, g = h / group;
      const int64_t n = std::max<int64_t>(0, std::min(seqlens[b], Lmax));
      kt.resize((size_t)d * std::max<int64_t>(n, 1));
      S.resize(std::max<int64_t>(n, 1));
      P.resize(std::max<int64_t>(n, 1));
      transpose(kc + (b * Hkv + g) * Lmax * d, n, d, kt.data());
      score_row(q + bh * d, kt.data(), n, d, n, scale, S.data(), total);
      double m, l;
      softmax_row(S.data(), P.data(), n, m, l);
      pv_row(P.data(), vc + (b * Hkv + g) * Lmax * dv, dv, dv, n, o + bh * dv, total);
      lse[bh] = (l > 0.0) ? m + std::log(l) : kNegInf;
    }
  }
  if (macs) *macs = total;
}

// Paged decode: pages [num_pages, Hkv, page, d]; logical key j of sequence b
// is row j % page of physical page table[b * max_pages + j / page].  The
// sequence's rows are gathered in logical order, then as oracle_decode.
void oracle_decode_paged(const double* q, const double* kp, const double* vp, const int64_t* table,
                         const int64_t* seqlens, int64_t B, int64_t H, int64_t Hkv, int64_t page, int64_t max_pages,
                         int64_t d, int64_t dv, double scale, double* o, double* lse, int64_t* macs) {
  const int64_t group = H / Hkv;
  int64_t total = 0;
#pragma omp parallel reduction(+ : total)
  {
    std::vector<double> kt, vg, S, P;
#pragma omp for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < B * H; ++bh) {
      const int64_t b = bh / H, h = bh % H, g = h / group;
      const int64_t n = std::max<int64_t>(0, std::min(seqlens[b], page * max_pages));
      const size_t n1 = (size_t)std::max<int64_t>(n, 1);
      kt.resize(d * n1);
      vg.resize(dv * n1);
      S.resize(n1);
      P.resize(n1);
      for (int64_t j = 0; j < n; ++j) {
        const int64_t pg = table[b * max_pages + j / page];
        const double* kr = kp + ((pg * Hkv + g) * page + j % page) * d;
        const double* vr = vp + ((pg * Hkv + g) * page + j % page) * dv;
        for (int64_t c = 0; c < d; ++c) kt[c * n + j] = kr[c];
        std::memcpy(vg.data() + j * dv, vr, sizeof(double) * dv);
      }
      score_row(q + bh * d, kt.data(), n, d, n, scale, S.data(), total);
      double m, l;
      softmax_row(S.data(), P.data(), n, m, l);
      pv_row(P.data(), vg.data(), dv, dv, n, o + bh * dv, total);
      lse[bh] = (l > 0.0) ? m + std::log(l) : kNegInf;
    }
  }
  if (macs) *macs = total;
}

// HSTU pointwise attention over packed sequences: q, k [T,H,d], v [T,H,dv],
// offsets [nseq+1]; sequence b owns rows [offsets[b], offsets[b+1]).  For
// each sequence, head and row i (local index), in the listing's order:
//   x_ij = sum_c q_ic k_jc;  x_ij *= alpha;  x_ij = x_ij / (1 + e^-x_ij);
//   x_ij *= mask_ij / n (mask: j <= i when causal, else 1; 1/n = inv_n);
//   O_i = sum_j x_ij v_j.
// o [T,H,dv] written (rows of every sequence).
void oracle_hstu_jagged(const double* q, const double* k, const double* v, const int64_t* offsets, int64_t nseq,
                        int64_t H, int64_t d, int64_t dv, double alpha, double inv_n, int causal, double* o,
                        int64_t* macs) {
  // tasks: (sequence, head, row panel)
  std::vector<int64_t> first(nseq + 1, 0);
  std::vector<int64_t> R(nseq);
  for (int64_t b = 0; b < nseq; ++b) {
    const int64_t L = std::max<int64_t>(0, offsets[b + 1] - offsets[b]);
    R[b] = panel_rows(L, L);
    first[b + 1] = first[b] + H * ((L + R[b] - 1) / R[b]);
  }
  const int64_t ntask = first[nseq];
  const int64_t rs = H * d, rsv = H * dv;  // elements between consecutive tokens
  int64_t total = 0;
#pragma omp parallel reduction(+ : total)
  {
    std::vector<double> kt, X;
    int64_t kt_key = -1;
#pragma omp for schedule(dynamic, 1)
    for (int64_t t = 0; t < ntask; ++t) {
      const int64_t b = std::upper_bound(first.begin(), first.end(), t) - first.begin() - 1;
      const int64_t s0 = offsets[b];
      const int64_t L = offsets[b + 1] - s0;
      const int64_t np = (L + R[b] - 1) / R[b];
      const int64_t h = (t - first[b]) / np;
      const int64_t p0 = ((t - first[b]) % np) * R[b];
      const int64_t pr = std::min(R[b], L - p0);
      if (kt_key != b * H + h) {
        kt.resize((size_t)d * L);
        for (int64_t j = 0; j < L; ++j)
          for (int64_t c = 0; c < d; ++c) kt[c * L + j] = k[(s0 + j) * rs + h * d + c];
        kt_key = b * H + h;
      }
      X.resize((size_t)R[b] * L);
      for (int64_t r = 0; r < pr; ++r) {
        const int64_t i = p0 + r;
        const int64_t nv = visible(i, L, causal);
        double* x = X.data() + r * L;
        // x = q k^T (the visible part; masked entries become 0 below)
        std::fill(x, x + L, 0.0);
        for (int64_t c = 0; c < d; ++c) {
          axpy(q[(s0 + i) * rs + h * d + c], kt.data() + c * L, x, nv);
          total += nv;
        }
        for (int64_t j = 0; j < nv; ++j) x[j] *= alpha;                    // x *= alpha
        for (int64_t j = 0; j < nv; ++j) x[j] = x[j] / (1.0 + std::exp(-x[j]));  // x = silu(x)
        for (int64_t j = 0; j < nv; ++j) x[j] *= inv_n;                    // x *= mask / n
        std::fill(x + nv, x + L, 0.0);
        // O = x V
        double* orow = o + (s0 + i) * rsv + h * dv;
        std::fill(orow, orow + dv, 0.0);
        for (int64_t j = 0; j < nv; ++j) {
          axpy(x[j], v + (s0 + j) * rsv + h * dv, orow, dv);
          total += dv;
        }
      }
    }
  }
  if (macs) *macs = total;
}

// Attention backward for a given dO.  q, dout [B,H,N,d]; k, v [B,Hkv,N,d].
// dq [B,H,N,d], dk, dv [B,Hkv,N,d] written.  One task per (batch, kv head):
// the kv head's gradients sum over the query heads of its group, in head
// order, then over row panels in row order, so no two threads touch one
// output element.  Per panel of query rows:
//   S, P (two-pass softmax) as in the forward;  dV += P^T dO;
//   dP = dO V^T;  D_i = sum_j P_ij dP_ij;  dS = P * (dP - D);
//   dQ = scale dS K;  dK += scale dS^T Q.
// macs counts the multiply-adds of the five products (S, dV, dP, dQ, dK).
void oracle_attention_backward(const double* q, const double* k, const double* v, const double* dout, int64_t B,
                               int64_t H, int64_t Hkv, int64_t N, int64_t d, double scale, int causal, double* dq,
                               double* dk, double* dv, int64_t* macs) {
  const int64_t group = H / Hkv;
  const int64_t R = panel_rows(N, N);
  int64_t total = 0;
  std::memset(dk, 0, sizeof(double) * B * Hkv * N * d);
  std::memset(dv, 0, sizeof(double) * B * Hkv * N * d);
#pragma omp parallel reduction(+ : total)
  {
    std::vector<double> kt((size_t)d * N), vt((size_t)d * N), S((size_t)R * N), P((size_t)R * N),
        dP((size_t)R * N), dS((size_t)R * N);
#pragma omp for schedule(dynamic, 1)
    for (int64_t bg = 0; bg < B * Hkv; ++bg) {
      const int64_t b = bg / Hkv, g = bg % Hkv;
      const double* kh = k + bg * N * d;
      const double* vh = v + bg * N * d;
      double* dkh = dk + bg * N * d;
      double* dvh = dv + bg * N * d;
      transpose(kh, N, d, kt.data());
      transpose(vh, N, d, vt.data());
      for (int64_t h = g * group; h < (g + 1) * group; ++h) {
        const int64_t bh = b * H + h;
        const double* qh = q + bh * N * d;
        const double* doh = dout + bh * N * d;
        double* dqh = dq + bh * N * d;
        for (int64_t p0 = 0; p0 < N; p0 += R) {
          const int64_t pr = std::min(R, N - p0);
          for (int64_t r = 0; r < pr; ++r) {
            const int64_t i = p0 + r;
            const int64_t nv = visible(i, N, causal);
            double* s = S.data() + r * N;
            double* p = P.data() + r * N;
            double* dp = dP.data() + r * N;
            double* ds = dS.data() + r * N;
            // S and P
            score_row(qh + i * d, kt.data(), N, d, nv, scale, s, total);
            double m, l;
            softmax_row(s, p, nv, m, l);
            // dP = dO V^T (row i)
            std::fill(dp, dp + nv, 0.0);
            for (int64_t c = 0; c < d; ++c) {
              axpy(doh[i * d + c], vt.data() + c * N, dp, nv);
              total += nv;
            }
            // D_i and dS
            double Di = 0.0;
            for (int64_t j = 0; j < nv; ++j) Di += p[j] * dp[j];
            for (int64_t j = 0; j < nv; ++j) ds[j] = p[j] * (dp[j] - Di);
            // dQ_i = scale sum_j dS_ij k_j
            double* dqi = dqh + i * d;
            std::fill(dqi, dqi + d, 0.0);
            for (int64_t j = 0; j < nv; ++j) {
              axpy(scale * ds[j], kh + j * d, dqi, d);
              total += d;
            }
          }
          // dV += P^T dO and dK += scale dS^T Q over the panel's rows, key by key
          for (int64_t j = 0; j < N; ++j) {
            for (int64_t r = 0; r < pr; ++r) {
              const int64_t i = p0 + r;
              if (j >= visible(i, N, causal)) continue;
              axpy(P[r * N + j], doh + i * d, dvh + j * d, d);
              axpy(scale * dS[r * N + j], qh + i * d, dkh + j * d, d);
              total += 2 * d;
            }
          }
        }
      }
    }
  }
  if (macs) *macs = total;
}

}  // extern "C"
