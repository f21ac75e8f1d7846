// CPU oracle of the mHC layer (Manifold-Constrained Hyper-Connections).
//
// TEST INFRASTRUCTURE ONLY.  The parity tests, the smoke check and the
// benchmark's CPU-baseline leg call it; the product path never does.  It
// shares no code, header, table or helper with the HIP library: plain,
// single-threaded C++17, every quantity in double, written from the pages'
// definitions, step by step and in their order, so it can be checked by eye.
//
// Sources (page title, then the section / equation / table used):
//  [P2] V. Dubrov, "DeepSeek mHC: Manifold-Constrained Hyper-Connections"
//       (slavadubrov.com, Dutch translation): sections "Kernmechanismen"
//       (update Eq. 3), "Het probleem van de samengestelde map" (composite
//       map, Amax Gain Magnitude), "Sinkhorn-Knopp-projectie" (procedure,
//       3x3 example, NumPy demo), "Details van de parameterisatie" (sigmoid
//       and 2*sigmoid maps).
//  [P5] "mHC" study notes on DeepSeek-V4 (t6page.pages.dev): equations
//       dsv4-mhc-hc-update, dsv4-mhc-rmsnorm, dsv4-mhc-a-tilde / b-tilde /
//       c-tilde, dsv4-mhc-sinkhorn-init, dsv4-mhc-sinkhorn, dsv4-mhc-gate;
//       table tbl-dsv4-mhc-mixed-precision.
//
// Readings where the pages leave a step open (each also listed in the design
// notes): RMSNorm epsilon is a parameter (the workloads use 1e-6) placed under
// the square root; RMSNorm has unit gain and runs over all n*d elements of the
// flattened state; phi's columns are ordered pre | res | post and Mat() is
// row-major with row = output stream; Sinkhorn normalises columns, then rows,
// in every one of t_max iterations, with plain division and no early exit;
// the composite map is H_L ... H_1 (each new layer multiplies from the left).
//
// The backward (gradients of <G, X'> + <D, h> for given G and D) is the chain
// rule of this forward in reverse; the pages state only that training uses a
// custom backward that recomputes the maps ([P5] mixed-precision table).  It
// is pinned by central finite differences of the all-double forward and by
// exact identities (column-shift invariance of Sinkhorn, the alpha = 0 closed
// form, Euler's theorem for the scale-invariant RMSNorm).
//
// Parity pins: Sinkhorn, gates, aggregation, mixing and Amax are pinned by the
// pages' worked examples and closed forms (see tests/test_oracle_pins.py).
// RMSNorm and the projection have no printed values on the pages; they are
// pinned by brute force in an independent formulation, one-hot projections and
// the alpha = 0 closed form.

#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

namespace {

// ---- storage formats --------------------------------------------------------
// dtype 0 = fp32, 1 = bf16 (stored as the upper 16 bits of an IEEE fp32).

double bf16_value(uint16_t bits) {
  uint32_t u = static_cast<uint32_t>(bits) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return static_cast<double>(f);
}

// Nearest bf16 to v, ties to even, rounded once from the double.
uint16_t bf16_round(double v) {
  if (std::isnan(v)) return 0x7FC0;
  const double a = std::fabs(v);
  uint16_t sign = std::signbit(v) ? 0x8000 : 0;
  if (a == 0.0) return sign;
  int e;
  std::frexp(a, &e);               // a = f * 2^e, f in [0.5, 1)
  int E = e - 1;                   // a = 1.xxx * 2^E
  if (E < -126) E = -126;          // subnormal range keeps the quantum fixed
  const double q = std::ldexp(1.0, E - 7);
  const double r = std::nearbyint(a / q) * q;   // default mode: ties to even
  if (r >= std::ldexp(1.0, 128)) return sign | 0x7F80;
  const float rf = static_cast<float>(r);       // exact: r has <= 8 significant bits
  uint32_t u;
  std::memcpy(&u, &rf, 4);
  return sign | static_cast<uint16_t>(u >> 16);
}

double load(int dtype, const void* base, int64_t i) {
  if (dtype == 0) return static_cast<double>(static_cast<const float*>(base)[i]);
  return bf16_value(static_cast<const uint16_t*>(base)[i]);
}

double store_round(int dtype, double v) {
  if (dtype == 0) return static_cast<double>(static_cast<float>(v));
  return bf16_value(bf16_round(v));
}

void store(int dtype, void* base, int64_t i, double v) {
  if (dtype == 0) static_cast<float*>(base)[i] = static_cast<float>(v);
  else static_cast<uint16_t*>(base)[i] = bf16_round(v);
}

double sigmoid(double u) { return 1.0 / (1.0 + std::exp(-u)); }

// ---- Sinkhorn-Knopp ([P2] Sinkhorn-Knopp-projectie; [P5] sinkhorn-init, sinkhorn)
// M0 = exp(logits); then t_max times: divide every column by its sum, then
// divide every row by its sum.  M is n x n row-major.
// trace (nullable) receives, for each iteration t and each half-step h
// (0 = after the column step, 1 = after the row step), the n row sums then the
// n column sums: trace[((t * 2 + h) * 2 + 0) * n + i] = row sum i,
//                trace[((t * 2 + h) * 2 + 1) * n + j] = column sum j.
void sinkhorn(int n, const double* logits, int t_max, double* M, double* trace) {
  for (int i = 0; i < n * n; ++i) M[i] = std::exp(logits[i]);
  std::vector<double> s(n);
  for (int t = 0; t < t_max; ++t) {
    for (int h = 0; h < 2; ++h) {
      if (h == 0) {
        for (int j = 0; j < n; ++j) {                    // column sums
          s[j] = 0.0;
          for (int i = 0; i < n; ++i) s[j] += M[i * n + j];
        }
        for (int i = 0; i < n; ++i)
          for (int j = 0; j < n; ++j) M[i * n + j] = M[i * n + j] / s[j];
      } else {
        for (int i = 0; i < n; ++i) {                    // row sums
          s[i] = 0.0;
          for (int j = 0; j < n; ++j) s[i] += M[i * n + j];
        }
        for (int i = 0; i < n; ++i)
          for (int j = 0; j < n; ++j) M[i * n + j] = M[i * n + j] / s[i];
      }
      if (trace) {
        double* tr = trace + static_cast<int64_t>(t * 2 + h) * 2 * n;
        for (int i = 0; i < n; ++i) {
          double rs = 0.0, cs = 0.0;
          for (int j = 0; j < n; ++j) { rs += M[i * n + j]; cs += M[j * n + i]; }
          tr[i] = rs;
          tr[n + i] = cs;
        }
      }
    }
  }
}

// ---- one token of the layer's map computation ([P5] rmsnorm, a/b/c-tilde, gate)
struct TokenMaps {
  double r = 0.0;                 // RMS of the flattened state
  std::vector<double> z;          // x_hat . phi, m values
  std::vector<double> logit;      // alpha * z + bias, m values
  std::vector<double> H;          // pre (n) | res (n*n) | post (n)
  double sk_err[4] = {0, 0, 0, 0};  // after the last column step: max|colsum-1|, max|rowsum-1|;
                                    // after the last row step:    max|colsum-1|, max|rowsum-1|
};

template <typename P>
TokenMaps token_maps(int n, int d, const std::vector<double>& x, const P* phi,
                     const P* bias, const P* alpha3, double eps, int t_max) {
  const int K = n * d;
  const int m = n * n + 2 * n;
  TokenMaps out;
  // RMSNorm of vec(X): x_hat = x / sqrt(mean(x^2) + eps), unit gain.
  double ss = 0.0;
  for (int k = 0; k < K; ++k) ss += x[k] * x[k];
  out.r = std::sqrt(ss / K + eps);
  std::vector<double> xh(K);
  for (int k = 0; k < K; ++k) xh[k] = x[k] / out.r;
  // Dynamic projection z = x_hat . phi   (phi is [K, m] row-major).
  out.z.assign(m, 0.0);
  for (int j = 0; j < m; ++j) {
    double acc = 0.0;
    for (int k = 0; k < K; ++k) acc += xh[k] * static_cast<double>(phi[static_cast<int64_t>(k) * m + j]);
    out.z[j] = acc;
  }
  // Scale by the block's alpha and add the static bias.
  out.logit.assign(m, 0.0);
  for (int j = 0; j < m; ++j) {
    const double a = (j < n) ? alpha3[0] : (j < n + n * n) ? alpha3[1] : alpha3[2];
    out.logit[j] = a * out.z[j] + static_cast<double>(bias[j]);
  }
  out.H.assign(m, 0.0);
  // Read map: sigmoid; write map: 2 * sigmoid.
  for (int i = 0; i < n; ++i) out.H[i] = sigmoid(out.logit[i]);
  for (int i = 0; i < n; ++i) out.H[n + n * n + i] = 2.0 * sigmoid(out.logit[n + n * n + i]);
  // Residual map: Sinkhorn-Knopp on exp(Mat(logits_res)).
  std::vector<double> trace(static_cast<size_t>(t_max) * 4 * n);
  sinkhorn(n, &out.logit[n], t_max, &out.H[n], t_max > 0 ? trace.data() : nullptr);
  if (t_max > 0) {
    for (int h = 0; h < 2; ++h) {
      const double* tr = trace.data() + static_cast<int64_t>((t_max - 1) * 2 + h) * 2 * n;
      double rerr = 0.0, cerr = 0.0;
      for (int i = 0; i < n; ++i) {
        rerr = std::fmax(rerr, std::fabs(tr[i] - 1.0));
        cerr = std::fmax(cerr, std::fabs(tr[n + i] - 1.0));
      }
      out.sk_err[2 * h + 0] = cerr;
      out.sk_err[2 * h + 1] = rerr;
    }
  }
  return out;
}

// ---- the HC form of the maps, for contrast ([P2] Kernmechanismen: in HC every
// map is a learned static part, a bias, plus an input-dependent term passed
// through tanh, so its values can take either sign; Details van de
// parameterisatie: mHC replaces that tanh by the sigmoid gates).  Reading:
// H = bias + alpha_blk * tanh(z) for all three maps, with z = x_hat . phi as
// in mHC and no Sinkhorn.
std::vector<double> hc_maps(int n, int d, const std::vector<double>& x, const float* phi, const float* bias,
                            const float* alpha3, double eps) {
  const int m = n * n + 2 * n;
  const TokenMaps tm = token_maps(n, d, x, phi, bias, alpha3, eps, 0);   // r and z only
  std::vector<double> H(m);
  for (int j = 0; j < m; ++j) {
    const int blk = (j < n) ? 0 : (j < n + n * n) ? 1 : 2;     // pre | res | post
    const double a = static_cast<double>(alpha3[blk]);
    H[j] = static_cast<double>(bias[j]) + a * std::tanh(tm.z[j]);
  }
  return H;
}

// The maps of one layer for one token: kind 0 = mHC, kind 1 = HC.
std::vector<double> layer_maps(int kind, int n, int d, const std::vector<double>& x, const float* phi,
                               const float* bias, const float* alpha3, double eps, int t_max, double* sk_err) {
  if (kind == 1) return hc_maps(n, d, x, phi, bias, alpha3, eps);
  TokenMaps tm = token_maps(n, d, x, phi, bias, alpha3, eps, t_max);
  if (sk_err) for (int j = 0; j < 4; ++j) sk_err[j] = tm.sk_err[j];
  return tm.H;
}

// Aggregation h = H_pre . X   ([P2] Kernmechanismen, Eq. 3: F(H_pre x_l)).
void aggregate(int n, int d, const std::vector<double>& x, const double* Hpre, double* h) {
  for (int c = 0; c < d; ++c) {
    double acc = 0.0;
    for (int i = 0; i < n; ++i) acc += Hpre[i] * x[static_cast<int64_t>(i) * d + c];
    h[c] = acc;
  }
}

// Mixing + broadcast-add X' = H_res X + H_post^T F   ([P2] Eq. 3; [P5] hc-update).
void mix(int n, int d, const std::vector<double>& x, const std::vector<double>& y,
         const double* Hres, const double* Hpost, double* xo) {
  for (int i = 0; i < n; ++i) {
    for (int c = 0; c < d; ++c) {
      double acc = 0.0;
      for (int j = 0; j < n; ++j) acc += Hres[i * n + j] * x[static_cast<int64_t>(j) * d + c];
      xo[static_cast<int64_t>(i) * d + c] = acc + Hpost[i] * y[c];
    }
  }
}

// ---- backward of one token (reading: the pages give no backward formulas, only
// that the layer is trained with a custom backward that recomputes the maps;
// this is the chain rule of the forward above, step by step in reverse).
// The differentiated quantity is L = <G, X'> + <D, h>: G is the gradient
// arriving at the layer output X' and D the gradient arriving at the sublayer
// input h, both taken as given (F stays outside the layer, as in the forward).

// Sinkhorn backward: forward again keeping every iterate, then reverse the
// 2 * t_max normalisations.  dM (n x n) enters as dL/dH_res and leaves as
// dL/dlogits_res.
void sinkhorn_backward(int n, const double* logits, int t_max, double* dM) {
  const int nn = n * n;
  // iter[s] is the matrix before normalisation s (s = 2t: column step of
  // iteration t, s = 2t + 1: its row step); sums[s] the divisors it used.
  std::vector<double> iter(static_cast<size_t>(2 * t_max + 1) * nn), sums(static_cast<size_t>(2 * t_max) * n);
  double* M0 = iter.data();
  for (int i = 0; i < nn; ++i) M0[i] = std::exp(logits[i]);
  for (int st = 0; st < 2 * t_max; ++st) {
    const double* A = iter.data() + static_cast<size_t>(st) * nn;
    double* B = iter.data() + static_cast<size_t>(st + 1) * nn;
    double* sm = sums.data() + static_cast<size_t>(st) * n;
    const bool col = (st % 2 == 0);
    for (int a = 0; a < n; ++a) {
      sm[a] = 0.0;
      for (int b = 0; b < n; ++b) sm[a] += col ? A[b * n + a] : A[a * n + b];
    }
    for (int i = 0; i < n; ++i)
      for (int j = 0; j < n; ++j) B[i * n + j] = A[i * n + j] / (col ? sm[j] : sm[i]);
  }
  // Reverse.  For B = A / s with s the sum of A's line (row or column):
  // dA = (dB - <dB, B> over that line) / s.
  std::vector<double> dA(nn);
  for (int st = 2 * t_max - 1; st >= 0; --st) {
    const double* B = iter.data() + static_cast<size_t>(st + 1) * nn;
    const double* sm = sums.data() + static_cast<size_t>(st) * n;
    const bool col = (st % 2 == 0);
    for (int a = 0; a < n; ++a) {
      double dot = 0.0;
      for (int b = 0; b < n; ++b) {
        const int e = col ? b * n + a : a * n + b;
        dot += dM[e] * B[e];
      }
      for (int b = 0; b < n; ++b) {
        const int e = col ? b * n + a : a * n + b;
        dA[e] = (dM[e] - dot) / sm[a];
      }
    }
    for (int i = 0; i < nn; ++i) dM[i] = dA[i];
  }
  // M0 = exp(logits)
  for (int i = 0; i < nn; ++i) dM[i] *= M0[i];
}

struct TokenGrads {
  std::vector<double> dx;       // K
  std::vector<double> dy;       // d
  std::vector<double> dH;       // m: dL/dH (pre | res | post)
  std::vector<double> dlogit;   // m
  std::vector<double> dz;       // m
  std::vector<double> xhat;     // K
  double dalpha[3] = {0, 0, 0};
};

template <typename P>
TokenGrads token_backward(int n, int d, const std::vector<double>& x, const std::vector<double>& y,
                          const P* phi, const P* bias, const P* alpha3, double eps, int t_max,
                          const std::vector<double>& G, const std::vector<double>& D) {
  const int K = n * d;
  const int m = n * n + 2 * n;
  const TokenMaps tm = token_maps(n, d, x, phi, bias, alpha3, eps, t_max);
  const double* Hpre = &tm.H[0];
  const double* Hres = &tm.H[n];
  const double* Hpost = &tm.H[n + n * n];
  TokenGrads g;
  g.dx.assign(K, 0.0);
  g.dy.assign(d, 0.0);
  g.dH.assign(m, 0.0);
  // Mixing + broadcast-add: X'_i = sum_j H_res[i][j] X_j + H_post[i] Y.
  for (int i = 0; i < n; ++i) {
    for (int j = 0; j < n; ++j) {
      double acc = 0.0;
      for (int c = 0; c < d; ++c) acc += G[i * d + c] * x[j * d + c];
      g.dH[n + i * n + j] = acc;
    }
    double acc = 0.0;
    for (int c = 0; c < d; ++c) acc += G[i * d + c] * y[c];
    g.dH[n + n * n + i] = acc;
  }
  for (int c = 0; c < d; ++c) {
    double acc = 0.0;
    for (int i = 0; i < n; ++i) acc += Hpost[i] * G[i * d + c];
    g.dy[c] = acc;
  }
  for (int j = 0; j < n; ++j)
    for (int c = 0; c < d; ++c) {
      double acc = 0.0;
      for (int i = 0; i < n; ++i) acc += Hres[i * n + j] * G[i * d + c];
      g.dx[j * d + c] += acc;
    }
  // Aggregation: h = sum_i H_pre[i] X_i.
  for (int i = 0; i < n; ++i) {
    double acc = 0.0;
    for (int c = 0; c < d; ++c) acc += D[c] * x[i * d + c];
    g.dH[i] = acc;
    for (int c = 0; c < d; ++c) g.dx[i * d + c] += Hpre[i] * D[c];
  }
  // Maps: sigmoid gates, 2 * sigmoid gate, Sinkhorn on exp(logits_res).
  g.dlogit.assign(m, 0.0);
  for (int i = 0; i < n; ++i) {
    const double sp = Hpre[i];
    g.dlogit[i] = g.dH[i] * sp * (1.0 - sp);
    const double sq = Hpost[i] / 2.0;
    g.dlogit[n + n * n + i] = g.dH[n + n * n + i] * 2.0 * sq * (1.0 - sq);
  }
  std::vector<double> dM(g.dH.begin() + n, g.dH.begin() + n + n * n);
  sinkhorn_backward(n, &tm.logit[n], t_max, dM.data());
  for (int e = 0; e < n * n; ++e) g.dlogit[n + e] = dM[e];
  // logits = alpha_blk * z + bias.
  g.dz.assign(m, 0.0);
  for (int j = 0; j < m; ++j) {
    const int blk = (j < n) ? 0 : (j < n + n * n) ? 1 : 2;
    g.dalpha[blk] += g.dlogit[j] * tm.z[j];
    g.dz[j] = static_cast<double>(alpha3[blk]) * g.dlogit[j];
  }
  // z = x_hat . phi with x_hat = x / r, r = sqrt(sum(x^2) / K + eps).
  g.xhat.assign(K, 0.0);
  for (int k = 0; k < K; ++k) g.xhat[k] = x[k] / tm.r;
  std::vector<double> dxh(K, 0.0);
  for (int k = 0; k < K; ++k) {
    double acc = 0.0;
    for (int j = 0; j < m; ++j) acc += static_cast<double>(phi[static_cast<int64_t>(k) * m + j]) * g.dz[j];
    dxh[k] = acc;
  }
  // dL/dr = -sum_k dxh_k x_k / r^2;  dr/dx_k = x_k / (K r).
  double dr = 0.0;
  for (int k = 0; k < K; ++k) dr -= dxh[k] * x[k] / (tm.r * tm.r);
  for (int k = 0; k < K; ++k) g.dx[k] += dxh[k] / tm.r + dr * x[k] / (K * tm.r);
  return g;
}

// Parameter gradients are sums over tokens: dphi = sum_t x_hat_t^T dz_t,
// dbias = sum_t dlogit_t, dalpha = sum_t (per-block <dlogit, z>).
void clear_param_grads(int K, int m, double* dphi, double* dbias, double* dalpha) {
  if (dphi) for (int64_t i = 0; i < static_cast<int64_t>(K) * m; ++i) dphi[i] = 0.0;
  if (dbias) for (int j = 0; j < m; ++j) dbias[j] = 0.0;
  if (dalpha) for (int j = 0; j < 3; ++j) dalpha[j] = 0.0;
}

void add_param_grads(const TokenGrads& tg, int K, int m, double* dphi, double* dbias, double* dalpha) {
  if (dphi)
    for (int k = 0; k < K; ++k)
      for (int j = 0; j < m; ++j) dphi[static_cast<int64_t>(k) * m + j] += tg.xhat[k] * tg.dz[j];
  if (dbias) for (int j = 0; j < m; ++j) dbias[j] += tg.dlogit[j];
  if (dalpha) for (int j = 0; j < 3; ++j) dalpha[j] += tg.dalpha[j];
}

// Composite map P = H_L ... H_1 and its Amax Gain Magnitude ([P2] samengestelde
// map: max absolute row sum (forward) and column sum (backward)).
template <typename Real>
void composite_amax(int n, int L, const Real* Hstack, int64_t layer_stride, int64_t row_off,
                    double* P, double* gfwd, double* gbwd) {
  const int m = n * n + 2 * n;
  std::vector<double> A(n * n), B(n * n);
  for (int i = 0; i < n * n; ++i) P[i] = (i / n == i % n) ? 1.0 : 0.0;
  for (int l = 0; l < L; ++l) {
    const Real* H = Hstack + l * layer_stride + row_off * m + n;
    for (int i = 0; i < n * n; ++i) A[i] = static_cast<double>(H[i]);
    for (int i = 0; i < n; ++i)
      for (int j = 0; j < n; ++j) {
        double acc = 0.0;
        for (int k = 0; k < n; ++k) acc += A[i * n + k] * P[k * n + j];
        B[i * n + j] = acc;
      }
    for (int i = 0; i < n * n; ++i) P[i] = B[i];
  }
  double f = 0.0, b = 0.0;
  for (int i = 0; i < n; ++i) {
    double rs = 0.0, cs = 0.0;
    for (int j = 0; j < n; ++j) { rs += std::fabs(P[i * n + j]); cs += std::fabs(P[j * n + i]); }
    f = std::fmax(f, rs);
    b = std::fmax(b, cs);
  }
  *gfwd = f;
  *gbwd = b;
}

// Synthetic sublayer of the stack workload: F(h) = 0.5 * GELU(h), exact erf form.
double gelu_half(double h) { return 0.5 * (0.5 * h * (1.0 + std::erf(h / std::sqrt(2.0)))); }

bool bad_shape(int64_t T, int n, int d, int dtype) {
  return T < 0 || n < 1 || n > 16 || d < 1 || (dtype != 0 && dtype != 1);
}

}  // namespace

extern "C" {

int mhcref_version(void) { return 3; }

// Rounding helpers exposed for the tests: round doubles to bf16 bits (RNE).
void mhcref_round_bf16(const double* in, uint16_t* out, int64_t count) {
  for (int64_t i = 0; i < count; ++i) out[i] = bf16_round(in[i]);
}

void mhcref_sinkhorn(int n, const double* logits, int t_max, double* out, double* trace) {
  sinkhorn(n, logits, t_max, out, trace);
}

// Layer maps and aggregation for the listed tokens.
//   X      [T, n, d] in the storage dtype; phi [n*d, m] fp32; bias [m] fp32;
//   alpha3 {alpha_pre, alpha_res, alpha_post}; tokens[ntok] indices into T.
//   Outputs (compact, one row per listed token, nullable except H):
//   h [ntok, d], H [ntok, m], r [ntok], z [ntok, m], logit [ntok, m], sk_err [ntok, 4].
int mhcref_pre(int64_t T, int n, int d, int dtype, const void* X, const float* phi,
               const float* bias, const float* alpha3, double eps, int t_max,
               const int64_t* tokens, int64_t ntok, double* h, double* H, double* r,
               double* z, double* logit, double* sk_err) {
  if (bad_shape(T, n, d, dtype) || t_max < 0 || !X || !phi || !bias || !alpha3 || !H) return -1;
  const int K = n * d;
  const int m = n * n + 2 * n;
  std::vector<double> x(K);
  for (int64_t q = 0; q < ntok; ++q) {
    const int64_t t = tokens[q];
    if (t < 0 || t >= T) return -2;
    for (int k = 0; k < K; ++k) x[k] = load(dtype, X, t * K + k);   // vec(X_t): stream i at [i*d, (i+1)*d)
    TokenMaps tm = token_maps(n, d, x, phi, bias, alpha3, eps, t_max);
    for (int j = 0; j < m; ++j) H[q * m + j] = tm.H[j];
    if (h) aggregate(n, d, x, tm.H.data(), h + q * d);
    if (r) r[q] = tm.r;
    if (z) for (int j = 0; j < m; ++j) z[q * m + j] = tm.z[j];
    if (logit) for (int j = 0; j < m; ++j) logit[q * m + j] = tm.logit[j];
    if (sk_err) for (int j = 0; j < 4; ++j) sk_err[q * 4 + j] = tm.sk_err[j];
  }
  return 0;
}

// Mixing + broadcast-add for the listed tokens.
//   X [T, n, d], Y [T, d] storage dtype; Hc [ntok, m] fp32 (row q belongs to tokens[q]).
//   Out Xo [ntok, n, d] in double.
int mhcref_post(int64_t T, int n, int d, int dtype, const void* X, const void* Y, const float* Hc,
                const int64_t* tokens, int64_t ntok, double* Xo) {
  if (bad_shape(T, n, d, dtype) || !X || !Y || !Hc || !Xo) return -1;
  const int K = n * d;
  const int m = n * n + 2 * n;
  std::vector<double> x(K), y(d), Hd(m);
  for (int64_t q = 0; q < ntok; ++q) {
    const int64_t t = tokens[q];
    if (t < 0 || t >= T) return -2;
    for (int k = 0; k < K; ++k) x[k] = load(dtype, X, t * K + k);
    for (int c = 0; c < d; ++c) y[c] = load(dtype, Y, t * d + c);
    for (int j = 0; j < m; ++j) Hd[j] = static_cast<double>(Hc[q * m + j]);
    mix(n, d, x, y, &Hd[n], &Hd[n + n * n], Xo + q * K);
  }
  return 0;
}

// Composite Amax over a stack of maps.  Hs [L, T, m] fp32 (or fp64 in the
// _f64 variant); outputs per listed token (nullable): amax, gain_fwd,
// gain_bwd, composite [ntok, n, n].
static int amax_impl(int64_t T, int n, int L, const void* Hs, bool f64, const int64_t* tokens,
                     int64_t ntok, double* amax, double* gfwd, double* gbwd, double* comp) {
  if (T < 0 || n < 1 || n > 16 || L < 0 || !Hs) return -1;
  const int m = n * n + 2 * n;
  std::vector<double> P(n * n);
  for (int64_t q = 0; q < ntok; ++q) {
    const int64_t t = tokens[q];
    if (t < 0 || t >= T) return -2;
    double f, b;
    if (f64) composite_amax<double>(n, L, static_cast<const double*>(Hs), T * m, t, P.data(), &f, &b);
    else composite_amax<float>(n, L, static_cast<const float*>(Hs), T * m, t, P.data(), &f, &b);
    if (gfwd) gfwd[q] = f;
    if (gbwd) gbwd[q] = b;
    if (amax) amax[q] = std::fmax(f, b);
    if (comp) for (int i = 0; i < n * n; ++i) comp[q * n * n + i] = P[i];
  }
  return 0;
}

int mhcref_amax(int64_t T, int n, int L, const float* Hs, const int64_t* tokens, int64_t ntok,
                double* amax, double* gfwd, double* gbwd, double* comp) {
  return amax_impl(T, n, L, Hs, false, tokens, ntok, amax, gfwd, gbwd, comp);
}

int mhcref_amax_f64(int64_t T, int n, int L, const double* Hs, const int64_t* tokens, int64_t ntok,
                    double* amax, double* gfwd, double* gbwd, double* comp) {
  return amax_impl(T, n, L, Hs, true, tokens, ntok, amax, gfwd, gbwd, comp);
}

// 0.5 * GELU(h) of storage-dtype values, out in double.
int mhcref_gelu_half(int64_t count, int dtype, const void* h, double* y) {
  if (count < 0 || (dtype != 0 && dtype != 1) || !h || !y) return -1;
  for (int64_t i = 0; i < count; ++i) y[i] = gelu_half(load(dtype, h, i));
  return 0;
}

// L-layer stack for the listed tokens: per layer, maps + aggregation, then
// Y = 0.5 GELU(h), then mixing; storage rounding mirrors what a device
// implementation stores between steps (h, Y and X_{l+1} in the storage dtype,
// the maps H in fp32, which is what the mixing step reads back).
//   X0 [T, n, d] storage; phis [L, n*d, m]; biases [L, m]; alphas [L, 3].
//   Outputs: Xf [ntok, n, d] storage dtype; Hs [L, ntok, m] fp32 (nullable);
//   amax / gfwd / gbwd [ntok] (nullable); sk_err [L, ntok, 4] (nullable).
static int stack_impl(int kind, int64_t T, int n, int d, int dtype, int L, const void* X0, const float* phis,
                      const float* biases, const float* alphas, double eps, int t_max,
                      const int64_t* tokens, int64_t ntok, void* Xf, float* Hs, double* amax,
                      double* gfwd, double* gbwd, double* sk_err) {
  if (bad_shape(T, n, d, dtype) || L < 0 || t_max < 0 || !X0 || !phis || !biases || !alphas || !Xf)
    return -1;
  const int K = n * d;
  const int m = n * n + 2 * n;
  std::vector<double> x(K), xo(K), h(d), y(d), Hr(m);
  std::vector<float> Hl(static_cast<size_t>(L) * m);
  for (int64_t q = 0; q < ntok; ++q) {
    const int64_t t = tokens[q];
    if (t < 0 || t >= T) return -2;
    for (int k = 0; k < K; ++k) x[k] = load(dtype, X0, t * K + k);
    for (int l = 0; l < L; ++l) {
      const float* phi = phis + static_cast<int64_t>(l) * K * m;
      double skl[4] = {0, 0, 0, 0};
      const std::vector<double> Hd = layer_maps(kind, n, d, x, phi, biases + l * m, alphas + 3 * l, eps, t_max, skl);
      if (sk_err) for (int j = 0; j < 4; ++j) sk_err[(static_cast<int64_t>(l) * ntok + q) * 4 + j] = skl[j];
      for (int j = 0; j < m; ++j) {
        Hl[l * m + j] = static_cast<float>(Hd[j]);
        Hr[j] = static_cast<double>(Hl[l * m + j]);
      }
      aggregate(n, d, x, Hd.data(), h.data());
      for (int c = 0; c < d; ++c) h[c] = store_round(dtype, h[c]);
      for (int c = 0; c < d; ++c) y[c] = store_round(dtype, gelu_half(h[c]));
      mix(n, d, x, y, &Hr[n], &Hr[n + n * n], xo.data());
      for (int k = 0; k < K; ++k) x[k] = store_round(dtype, xo[k]);
    }
    for (int k = 0; k < K; ++k) store(dtype, Xf, q * K + k, x[k]);
    if (Hs) for (int l = 0; l < L; ++l) for (int j = 0; j < m; ++j) Hs[(static_cast<int64_t>(l) * ntok + q) * m + j] = Hl[l * m + j];
    if (amax || gfwd || gbwd) {
      std::vector<double> P(n * n);
      double f, b;
      composite_amax<float>(n, L, Hl.data(), m, 0, P.data(), &f, &b);
      if (gfwd) gfwd[q] = f;
      if (gbwd) gbwd[q] = b;
      if (amax) amax[q] = std::fmax(f, b);
    }
  }
  return 0;
}

int mhcref_stack(int64_t T, int n, int d, int dtype, int L, const void* X0, const float* phis,
                 const float* biases, const float* alphas, double eps, int t_max,
                 const int64_t* tokens, int64_t ntok, void* Xf, float* Hs, double* amax,
                 double* gfwd, double* gbwd, double* sk_err) {
  return stack_impl(0, T, n, d, dtype, L, X0, phis, biases, alphas, eps, t_max, tokens, ntok, Xf, Hs, amax, gfwd,
                    gbwd, sk_err);
}

// The same stack with the HC form of the maps (no Sinkhorn, no gates).
int mhcref_stack_hc(int64_t T, int n, int d, int dtype, int L, const void* X0, const float* phis,
                    const float* biases, const float* alphas, double eps, const int64_t* tokens, int64_t ntok,
                    void* Xf, float* Hs, double* amax, double* gfwd, double* gbwd) {
  return stack_impl(1, T, n, d, dtype, L, X0, phis, biases, alphas, eps, 0, tokens, ntok, Xf, Hs, amax, gfwd, gbwd,
                    nullptr);
}

// HC-form maps and aggregation for the listed tokens (outputs as mhcref_pre's H and h).
int mhcref_pre_hc(int64_t T, int n, int d, int dtype, const void* X, const float* phi, const float* bias,
                  const float* alpha3, double eps, const int64_t* tokens, int64_t ntok, double* h, double* H) {
  if (bad_shape(T, n, d, dtype) || !X || !phi || !bias || !alpha3 || !H) return -1;
  const int K = n * d;
  const int m = n * n + 2 * n;
  std::vector<double> x(K);
  for (int64_t q = 0; q < ntok; ++q) {
    const int64_t t = tokens[q];
    if (t < 0 || t >= T) return -2;
    for (int k = 0; k < K; ++k) x[k] = load(dtype, X, t * K + k);
    const std::vector<double> Hd = hc_maps(n, d, x, phi, bias, alpha3, eps);
    for (int j = 0; j < m; ++j) H[q * m + j] = Hd[j];
    if (h) aggregate(n, d, x, Hd.data(), h + q * d);
  }
  return 0;
}

// ---- backward ---------------------------------------------------------------
// Gradients of L = sum_t <G_t, X'_t> + <D_t, h_t> for the listed tokens.
//   X, G [T, n, d]; Y, D [T, d] in the storage dtype; phi [n*d, m], bias [m],
//   alpha3 [3] fp32.  Outputs in double: dX [ntok, n, d], dY [ntok, d],
//   dH [ntok, m] (nullable), dlogit [ntok, m] (nullable); dphi [n*d, m],
//   dbias [m] and dalpha [3] (nullable) are sums over the listed tokens.
int mhcref_bwd(int64_t T, int n, int d, int dtype, const void* X, const void* Y, const float* phi,
               const float* bias, const float* alpha3, double eps, int t_max, const void* G,
               const void* D, const int64_t* tokens, int64_t ntok, double* dX, double* dY, double* dH,
               double* dlogit, double* dphi, double* dbias, double* dalpha) {
  if (bad_shape(T, n, d, dtype) || t_max < 0 || !X || !Y || !phi || !bias || !alpha3 || !G || !D ||
      !dX || !dY)
    return -1;
  const int K = n * d;
  const int m = n * n + 2 * n;
  clear_param_grads(K, m, dphi, dbias, dalpha);
  std::vector<double> x(K), g(K), y(d), dd(d);
  for (int64_t q = 0; q < ntok; ++q) {
    const int64_t t = tokens[q];
    if (t < 0 || t >= T) return -2;
    for (int k = 0; k < K; ++k) { x[k] = load(dtype, X, t * K + k); g[k] = load(dtype, G, t * K + k); }
    for (int c = 0; c < d; ++c) { y[c] = load(dtype, Y, t * d + c); dd[c] = load(dtype, D, t * d + c); }
    const TokenGrads tg = token_backward(n, d, x, y, phi, bias, alpha3, eps, t_max, g, dd);
    for (int k = 0; k < K; ++k) dX[q * K + k] = tg.dx[k];
    for (int c = 0; c < d; ++c) dY[q * d + c] = tg.dy[c];
    if (dH) for (int j = 0; j < m; ++j) dH[q * m + j] = tg.dH[j];
    if (dlogit) for (int j = 0; j < m; ++j) dlogit[q * m + j] = tg.dlogit[j];
    add_param_grads(tg, K, m, dphi, dbias, dalpha);
  }
  return 0;
}

// The same layer entirely in double (inputs, parameters, outputs; no storage
// rounding), for the finite-difference checks of the backward.
//   X [T, n, d], Y [T, d], phi [n*d, m], bias [m], alpha3 [3]; outputs
//   h [T, d] and Xo [T, n, d].
int mhcref_layer_f64(int64_t T, int n, int d, const double* X, const double* Y, const double* phi,
                     const double* bias, const double* alpha3, double eps, int t_max, double* h,
                     double* Xo) {
  if (bad_shape(T, n, d, 0) || t_max < 0 || !X || !Y || !phi || !bias || !alpha3 || !h || !Xo) return -1;
  const int K = n * d;
  std::vector<double> x(K), y(d);
  for (int64_t t = 0; t < T; ++t) {
    for (int k = 0; k < K; ++k) x[k] = X[t * K + k];
    for (int c = 0; c < d; ++c) y[c] = Y[t * d + c];
    const TokenMaps tm = token_maps(n, d, x, phi, bias, alpha3, eps, t_max);
    aggregate(n, d, x, tm.H.data(), h + t * d);
    mix(n, d, x, y, &tm.H[n], &tm.H[n + n * n], Xo + t * K);
  }
  return 0;
}

// Backward of mhcref_layer_f64 over all T tokens (same outputs as mhcref_bwd).
int mhcref_bwd_f64(int64_t T, int n, int d, const double* X, const double* Y, const double* phi,
                   const double* bias, const double* alpha3, double eps, int t_max, const double* G,
                   const double* D, double* dX, double* dY, double* dH, double* dlogit, double* dphi,
                   double* dbias, double* dalpha) {
  if (bad_shape(T, n, d, 0) || t_max < 0 || !X || !Y || !phi || !bias || !alpha3 || !G || !D || !dX || !dY)
    return -1;
  const int K = n * d;
  const int m = n * n + 2 * n;
  clear_param_grads(K, m, dphi, dbias, dalpha);
  std::vector<double> x(K), g(K), y(d), dd(d);
  for (int64_t t = 0; t < T; ++t) {
    for (int k = 0; k < K; ++k) { x[k] = X[t * K + k]; g[k] = G[t * K + k]; }
    for (int c = 0; c < d; ++c) { y[c] = Y[t * d + c]; dd[c] = D[t * d + c]; }
    const TokenGrads tg = token_backward(n, d, x, y, phi, bias, alpha3, eps, t_max, g, dd);
    for (int k = 0; k < K; ++k) dX[t * K + k] = tg.dx[k];
    for (int c = 0; c < d; ++c) dY[t * d + c] = tg.dy[c];
    if (dH) for (int j = 0; j < m; ++j) dH[t * m + j] = tg.dH[j];
    if (dlogit) for (int j = 0; j < m; ++j) dlogit[t * m + j] = tg.dlogit[j];
    add_param_grads(tg, K, m, dphi, dbias, dalpha);
  }
  return 0;
}

}  // extern "C"
