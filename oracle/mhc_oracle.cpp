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

TokenMaps token_maps(int n, int d, const std::vector<double>& x, const float* phi,
                     const float* bias, const float* alpha3, double eps, int t_max) {
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

int mhcref_version(void) { return 1; }

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
int mhcref_stack(int64_t T, int n, int d, int dtype, int L, const void* X0, const float* phis,
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
      TokenMaps tm = token_maps(n, d, x, phi, biases + l * m, alphas + 3 * l, eps, t_max);
      if (sk_err) for (int j = 0; j < 4; ++j) sk_err[(static_cast<int64_t>(l) * ntok + q) * 4 + j] = tm.sk_err[j];
      for (int j = 0; j < m; ++j) {
        Hl[l * m + j] = static_cast<float>(tm.H[j]);
        Hr[j] = static_cast<double>(Hl[l * m + j]);
      }
      aggregate(n, d, x, tm.H.data(), h.data());
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

}  // extern "C"
