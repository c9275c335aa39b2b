// Plain, slow, obviously-correct CPU oracle for causal multi-head scaled
// dot-product self-attention and its training backward, in float64.
//
// TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
// bench's cpu_baseline leg may load this library.  It shares no code, header,
// table or helper with the GPU library; the two meet only through the seeded
// input generator.
//
// What it computes, per (b, h) slice independently (multi-head: the heads
// run side by side, "Let's build GPT" summary page, timestamp 1:22:27):
//   s_ij  = scale * <q_i, k_j>                 affinity = query . key of the
//                                              earlier tokens (1:04:00-1:06:16),
//                                              divided by sqrt(head size) (1:17:18)
//   mask  : entries above the diagonal are -inf, the diagonal is kept
//           (lower-triangular tril, 48:54; -inf fill, 55:20)
//   p_ij  = softmax over the row (rows sum to one, 51:04; softmax, 55:20)
//   o_i   = sum_j p_ij v_j                      (value is what is passed on, 1:10:15)
//   lse_i = log sum_{j<=i} exp(s_ij)            (natural log; extra output)
// Backward (the pages only say the model is trained by backprop; the
// formulas below are the chain rule applied to the forward above):
//   D_i   = <dO_i, o_i>
//   dP_ij = <dO_i, v_j>,  dS_ij = p_ij (dP_ij - D_i)
//   dV_j  = sum_{i>=j} p_ij dO_i
//   dQ_i  = scale * sum_{j<=i} dS_ij k_j
//   dK_j  = scale * sum_{i>=j} dS_ij q_i
// Layout: contiguous (B, H, T, hs), hs innermost; lse (B, H, T).
// gattn_ref_fwd_kv: the forward of the newest Tq tokens of a Tk-token
// sequence (q for those tokens, k and v for all of them); the pages' generate
// recomputes the whole forward per token instead (no key/value cache,
// "nanoGPT" notes section 5), whose last rows this equals.
// The full probability matrix is kept per slice: no recompute, no blocking.

#include <algorithm>
#include <cmath>
#include <cstddef>
#include <limits>
#include <thread>
#include <vector>

namespace {

struct Slice {
  const double* q;
  const double* k;
  const double* v;
  const double* dO;  // may be null (forward only)
  double* o;
  double* lse;
  double* dq;
  double* dk;
  double* dv;
};

double dot(const double* a, const double* b, int n) {
  double s = 0.0;
  for (int d = 0; d < n; ++d) s += a[d] * b[d];
  return s;
}

// Forward for one slice; fills p (T x T, row-major, zeros above the diagonal).
void forward_slice(const Slice& x, int T, int hs, double scale, std::vector<double>& p) {
  const double neg_inf = -std::numeric_limits<double>::infinity();
  std::vector<double> s(T);
  for (int i = 0; i < T; ++i) {
    double m = neg_inf;
    for (int j = 0; j < T; ++j) {
      s[j] = (j <= i) ? scale * dot(x.q + (size_t)i * hs, x.k + (size_t)j * hs, hs) : neg_inf;
      m = std::max(m, s[j]);
    }
    double z = 0.0;
    for (int j = 0; j <= i; ++j) z += std::exp(s[j] - m);
    double* prow = p.data() + (size_t)i * T;
    for (int j = 0; j < T; ++j) prow[j] = (j <= i) ? std::exp(s[j] - m) / z : 0.0;
    double* orow = x.o + (size_t)i * hs;
    for (int d = 0; d < hs; ++d) {
      double acc = 0.0;
      for (int j = 0; j <= i; ++j) acc += prow[j] * x.v[(size_t)j * hs + d];
      orow[d] = acc;
    }
    if (x.lse) x.lse[i] = m + std::log(z);
  }
}

void backward_slice(const Slice& x, int T, int hs, double scale, const std::vector<double>& p) {
  std::vector<double> D(T), ds((size_t)T * T, 0.0);
  for (int i = 0; i < T; ++i) D[i] = dot(x.dO + (size_t)i * hs, x.o + (size_t)i * hs, hs);
  for (int i = 0; i < T; ++i)
    for (int j = 0; j <= i; ++j) {
      double dp = dot(x.dO + (size_t)i * hs, x.v + (size_t)j * hs, hs);
      ds[(size_t)i * T + j] = p[(size_t)i * T + j] * (dp - D[i]);
    }
  for (int j = 0; j < T; ++j)
    for (int d = 0; d < hs; ++d) {
      double av = 0.0, ak = 0.0;
      for (int i = j; i < T; ++i) {
        av += p[(size_t)i * T + j] * x.dO[(size_t)i * hs + d];
        ak += ds[(size_t)i * T + j] * x.q[(size_t)i * hs + d];
      }
      x.dv[(size_t)j * hs + d] = av;
      x.dk[(size_t)j * hs + d] = scale * ak;
    }
  for (int i = 0; i < T; ++i)
    for (int d = 0; d < hs; ++d) {
      double aq = 0.0;
      for (int j = 0; j <= i; ++j) aq += ds[(size_t)i * T + j] * x.k[(size_t)j * hs + d];
      x.dq[(size_t)i * hs + d] = scale * aq;
    }
}

// Forward of Tq queries against Tk >= Tq keys for one slice: query i is the
// token at position Tk - Tq + i of the key sequence (the newest Tq tokens)
// and sees keys j <= Tk - Tq + i.  Same arithmetic, in the same order, as
// forward_slice for each row.
void forward_slice_kv(const double* q, const double* k, const double* v, double* o, double* lse,
                      int Tq, int Tk, int hs, double scale) {
  const double neg_inf = -std::numeric_limits<double>::infinity();
  const int off = Tk - Tq;
  std::vector<double> s(Tk), p(Tk);
  for (int i = 0; i < Tq; ++i) {
    const int last = off + i;  // newest visible key
    double m = neg_inf;
    for (int j = 0; j < Tk; ++j) {
      s[j] = (j <= last) ? scale * dot(q + (size_t)i * hs, k + (size_t)j * hs, hs) : neg_inf;
      m = std::max(m, s[j]);
    }
    double z = 0.0;
    for (int j = 0; j <= last; ++j) z += std::exp(s[j] - m);
    for (int j = 0; j < Tk; ++j) p[j] = (j <= last) ? std::exp(s[j] - m) / z : 0.0;
    double* orow = o + (size_t)i * hs;
    for (int d = 0; d < hs; ++d) {
      double acc = 0.0;
      for (int j = 0; j <= last; ++j) acc += p[j] * v[(size_t)j * hs + d];
      orow[d] = acc;
    }
    if (lse) lse[i] = m + std::log(z);
  }
}

template <class F>
void parallel_slices(int nslices, int nthreads, F&& f) {
  if (nthreads <= 0) nthreads = (int)std::max(1u, std::thread::hardware_concurrency());
  nthreads = std::min(nthreads, std::max(1, nslices));
  std::vector<std::thread> pool;
  for (int t = 0; t < nthreads; ++t)
    pool.emplace_back([&, t] {
      for (int s = t; s < nslices; s += nthreads) f(s);
    });
  for (auto& th : pool) th.join();
}

}  // namespace

extern "C" {

int gattn_ref_hardware_threads(void) {
  return (int)std::max(1u, std::thread::hardware_concurrency());
}

// Forward.  o: (B,H,T,hs); lse: (B,H,T), may be null.  nthreads <= 0: all cores.
void gattn_ref_fwd(const double* q, const double* k, const double* v, double* o, double* lse,
                   int B, int H, int T, int hs, double scale, int nthreads) {
  const size_t st = (size_t)T * hs;
  parallel_slices(B * H, nthreads, [&](int s) {
    Slice x{q + s * st, k + s * st, v + s * st, nullptr, o + s * st,
            lse ? lse + (size_t)s * T : nullptr, nullptr, nullptr, nullptr};
    std::vector<double> p((size_t)T * T);
    forward_slice(x, T, hs, scale, p);
  });
}

// Forward of the newest Tq tokens against Tk >= Tq keys (decoding with the
// keys and values of earlier tokens kept): q, o (B,H,Tq,hs); k, v (B,H,Tk,hs);
// lse (B,H,Tq), may be null.  Query i sees keys j <= Tk - Tq + i.
void gattn_ref_fwd_kv(const double* q, const double* k, const double* v, double* o, double* lse,
                      int B, int H, int Tq, int Tk, int hs, double scale, int nthreads) {
  const size_t sq = (size_t)Tq * hs, sk = (size_t)Tk * hs;
  parallel_slices(B * H, nthreads, [&](int s) {
    forward_slice_kv(q + s * sq, k + s * sk, v + s * sk, o + s * sq,
                     lse ? lse + (size_t)s * Tq : nullptr, Tq, Tk, hs, scale);
  });
}

// Backward (recomputes the forward itself): writes dq, dk, dv and also o, lse.
void gattn_ref_bwd(const double* q, const double* k, const double* v, const double* dO,
                   double* dq, double* dk, double* dv, double* o, double* lse,
                   int B, int H, int T, int hs, double scale, int nthreads) {
  const size_t st = (size_t)T * hs;
  parallel_slices(B * H, nthreads, [&](int s) {
    Slice x{q + s * st, k + s * st, v + s * st, dO + s * st, o + s * st,
            lse + (size_t)s * T, dq + s * st, dk + s * st, dv + s * st};
    std::vector<double> p((size_t)T * T);
    forward_slice(x, T, hs, scale, p);
    backward_slice(x, T, hs, scale, p);
  });
}

}  // extern "C"
