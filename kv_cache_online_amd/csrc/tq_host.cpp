// Host side of libtq: Lloyd-Max codebook, matrix precomputation, argument
// validation and the extern "C" entry points declared in tq.h.
//
// Sources: ast-softpro.ru, "Технология TurboQuant и её применение с локальными
// LLM", section 1.2 "Как работает TurboQuant" (stage 1: random orthogonal
// rotation and a b-1 bit MSE-optimal Lloyd-Max quantizer per coordinate;
// stage 2: sign of a Gaussian projection of the residual, plus ||r||_2);
// kiosknews.app, "3 бита вместо 16: разбираем TurboQuant и когда его реально
// стоит включать", section "Как работает TurboQuant" (the codebook is computed
// once for the known post-rotation distribution and stored).

#include <cmath>
#include <cstring>
#include <vector>

#include <hip/hip_runtime_api.h>

#include "tq_common.h"

namespace {

// --------------------------------------------------------------- Lloyd-Max --
// Standard normal density and the probability of a cell [a, b), taken on the
// side of the smaller tail so that cells far out keep full relative precision.
double npdf(double x) {
  if (std::isinf(x)) return 0.0;
  return std::exp(-0.5 * x * x) * 0.39894228040143267794;  // 1/sqrt(2 pi)
}
double upper_tail(double x) {  // P(X >= x)
  if (x == INFINITY) return 0.0;
  if (x == -INFINITY) return 1.0;
  return 0.5 * std::erfc(x * 0.70710678118654752440);
}
double cell_prob(double a, double b) {
  if (a > 0) return upper_tail(a) - upper_tail(b);
  return upper_tail(-b) - upper_tail(-a);  // P(-b < X <= -a) by symmetry
}

uint16_t bf16_rne(double v) {
  float f = static_cast<float>(v);  // v is exactly representable or a remainder
  uint32_t u;
  std::memcpy(&u, &f, 4);
  uint32_t lsb = (u >> 16) & 1u;
  return static_cast<uint16_t>((u + 0x7FFFu + lsb) >> 16);
}
double bf16_val(uint16_t b) {
  uint32_t u = static_cast<uint32_t>(b) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

void split3(float v, uint16_t *hi, uint16_t *mid, uint16_t *lo) {
  double r = v;
  *hi = bf16_rne(r);
  r -= bf16_val(*hi);
  *mid = bf16_rne(r);
  r -= bf16_val(*mid);
  *lo = bf16_rne(r);
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool supported_d(int d) { return d == 64 || d == 128 || d == 256; }

int check_spec(const tq_tensor_spec &s, int d) {
  if (s.bits_mse < 1 || s.bits_mse > 3) return TQ_ERR_INVALID_ARG;
  if (s.sketch != 0 && s.sketch != 1) return TQ_ERR_INVALID_ARG;
  if (s.cb.bits_mse != s.bits_mse || s.cb.levels != (1 << s.bits_mse)) return TQ_ERR_INVALID_ARG;
  (void)d;
  return TQ_OK;
}

int check_config(const tq_config *cfg) {
  if (!cfg) return TQ_ERR_INVALID_ARG;
  if (cfg->d <= 0 || cfg->m != cfg->d) return TQ_ERR_INVALID_ARG;
  if (!supported_d(cfg->d)) return TQ_ERR_UNSUPPORTED;
  if (cfg->n_kv_heads <= 0 || cfg->n_q_heads <= 0 || cfg->n_q_heads % cfg->n_kv_heads)
    return TQ_ERR_INVALID_ARG;
  if (!cfg->rot || !cfg->proj || !cfg->prep) return TQ_ERR_INVALID_ARG;
  if (!aligned16(cfg->rot) || !aligned16(cfg->proj) || !aligned16(cfg->prep)) return TQ_ERR_INVALID_ARG;
  int e = check_spec(cfg->k, cfg->d);
  if (e) return e;
  return check_spec(cfg->v, cfg->d);
}

int check_cache(const tq_cache *c, const tq_tensor_spec &s) {
  if (!c || !c->idx || !c->scl) return TQ_ERR_INVALID_ARG;
  if (s.sketch && !c->sgn) return TQ_ERR_INVALID_ARG;
  if (c->capacity <= 0 || c->capacity % 32) return TQ_ERR_INVALID_ARG;
  if (c->layout != TQ_LAYOUT_TOKEN_MAJOR && c->layout != TQ_LAYOUT_BLOCK32) return TQ_ERR_INVALID_ARG;
  if (!aligned16(c->idx) || !aligned16(c->scl) || (c->sgn && !aligned16(c->sgn))) return TQ_ERR_INVALID_ARG;
  return TQ_OK;
}

tq::CodebookF32 cb_f32(const tq_codebook &cb) {
  tq::CodebookF32 o{};
  for (int i = 0; i < TQ_MAX_LEVELS - 1; ++i) o.thr[i] = cb.boundary_f32[i];
  for (int i = 0; i < TQ_MAX_LEVELS; ++i) o.cen[i] = cb.centroid_f32[i];
  o.levels = cb.levels;
  return o;
}

// The matrix-core quantize decides cells from |u| and the upper half of the
// codebook, which needs c[L-1-i] == -c[i] and t[L-2-i] == -t[i] in fp32.
bool cb_symmetric(const tq::CodebookF32 &c) {
  const int L = c.levels;
  for (int i = 0; i < L; ++i)
    if (c.cen[L - 1 - i] != -c.cen[i]) return false;
  for (int i = 0; i + 1 < L; ++i)
    if (c.thr[L - 2 - i] != -c.thr[i]) return false;
  return true;
}

}  // namespace

namespace tq {

DecodePlan decode_plan(const tq_config &cfg, int32_t batch, int32_t max_len) {
  DecodePlan p{};
  const int G = cfg.n_kv_heads > 0 ? cfg.n_q_heads / cfg.n_kv_heads : 1;
  p.fast = (cfg.d == 128 || cfg.d == 256) && (G == 4 || G == 8);
  p.rb = G >= 4 ? G / 4 : 1;
  // Split length: a multiple of 256 slots (4 waves x 64), sized for about 512
  // work-groups (two per CU), at most 1280 slots (five key tiles per wave, whose
  // scores the split pass keeps in registers).  Where the grid holds many more
  // work-groups than the chip runs at once, the longest split is the fastest:
  // each work-group has a fixed cost (query operands, the split maximum, its
  // partial) and the merge reads one partial per split.
  const int64_t pairs = int64_t(batch) * cfg.n_kv_heads;
  int64_t st = pairs > 0 ? (int64_t(max_len) * pairs + 511) / 512 : 256;
  st = (st + 255) / 256 * 256;
  if (st > 1280) st = 1280;
  if (st < 256) st = 256;
  p.split_tokens = static_cast<int32_t>(st);
  // Splits are aligned to absolute 64-slot tiles, so a sequence may start up to 63
  // slots into its first split.
  p.n_split = static_cast<int32_t>((int64_t(max_len) + 63 + st - 1) / st);
  if (p.n_split < 1) p.n_split = 1;
  if (p.n_split > 2048) p.fast = 0;  // the matrix-core merge keeps one weight per split in LDS
  p.part_stride = 4 + cfg.d + cfg.m;  // the matrix-core records (m, l, pad, pad, A, B); the reference kernels use fewer
  const size_t nq = size_t(batch) * cfg.n_q_heads;
  const size_t nkv = size_t(batch) * cfg.n_kv_heads;
  size_t o = 0;
  p.off_qr = o;     o = align256(o + nq * cfg.d * 4);
  p.off_qs = o;     o = align256(o + nq * cfg.m * 4);
  p.off_part = o;   o = align256(o + nq * size_t(p.n_split) * p.part_stride * 4);
  p.off_qop = o;    o = align256(o + nkv * q_operand_bytes(cfg.d, G >= 1 && G <= 16 ? G : 16));
  p.off_qscale = o; o = align256(o + nkv * q_scale_bytes());
  p.off_smax = o;   o = align256(o + nq * size_t(p.n_split) * 4);
  p.total = o;
  return p;
}

}  // namespace tq

extern "C" {

const char *tq_status_string(int s) {
  switch (s) {
    case TQ_OK: return "ok";
    case TQ_ERR_INVALID_ARG: return "invalid argument";
    case TQ_ERR_UNSUPPORTED: return "unsupported configuration";
    case TQ_ERR_WORKSPACE: return "workspace too small";
    case TQ_ERR_LAUNCH: return "kernel launch failed";
    case TQ_ERR_NO_CONVERGENCE: return "Lloyd-Max did not converge";
    default: return "unknown status";
  }
}

namespace {

// Fill *out from an antisymmetric codebook in absolute units: centroids cs[L],
// interior boundaries the midpoints, plus fp32 copies and the Walsh
// expansion over index bit-planes: walsh[S] = mean_i c[i] prod_{p in S} s_p(i).
// Code L-1-i has every bit of i flipped and c[L-1-i] = -c[i], so the pair
// (i, L-1-i) cancels for even |S| and doubles for odd |S|.
void finish_codebook(int bits_mse, double sigma, const double *cs, double mse, int iterations, tq_codebook *out) {
  const int L = 1 << bits_mse;
  std::memset(out, 0, sizeof(*out));
  out->bits_mse = bits_mse;
  out->levels = L;
  out->sigma = sigma;
  for (int k = 0; k < L; ++k) {
    out->centroid[k] = cs[k];
    out->centroid_f32[k] = static_cast<float>(cs[k]);
  }
  for (int k = 0; k + 1 < L; ++k) {
    out->boundary[k] = 0.5 * (cs[k] + cs[k + 1]);
    out->boundary_f32[k] = static_cast<float>(out->boundary[k]);
  }
  for (int S = 0; S < L; ++S) {
    if (!(__builtin_popcount(S) & 1)) {
      out->walsh[S] = 0.0;
      continue;
    }
    double acc = 0.0;
    for (int i = 0; i < L / 2; ++i) {
      double sgn = 1.0;
      for (int p = 0; p < bits_mse; ++p)
        if (S >> p & 1) sgn *= (i >> p & 1) ? 1.0 : -1.0;
      acc += out->centroid[i] * sgn;
    }
    out->walsh[S] = 2.0 * acc / L;
  }
  out->mse = mse;
  out->iterations = iterations;
}

// ------------------------------------------ exact law of one sphere coordinate --
// A coordinate u of a uniformly random unit vector in R^d (d >= 3) has density
// (1 - u^2)^((d-3)/2) / B(1/2, (d-1)/2) on [-1, 1]: u^2 ~ Beta(1/2, (d-1)/2).

// Regularized incomplete beta I_x(p, q): prefactor x^p (1-x)^q / (p B(p, q))
// over the continued fraction 1 + d1/(1 + d2/(1 + ...)) with
// d_{2m+1} = -(p+m)(p+q+m) x / ((p+2m)(p+2m+1)), d_{2m} = m(q-m) x / ((p+2m-1)(p+2m)),
// evaluated with the modified Lentz method; past x = (p+1)/(p+q+2), where the
// fraction converges slowly, through I_x(p, q) = 1 - I_{1-x}(q, p).
double betainc_reg(double p, double q, double x) {
  if (x <= 0.0) return 0.0;
  if (x >= 1.0) return 1.0;
  if (x > (p + 1.0) / (p + q + 2.0)) return 1.0 - betainc_reg(q, p, 1.0 - x);
  const double lnpre = p * std::log(x) + q * std::log1p(-x) - std::log(p) -
                       (std::lgamma(p) + std::lgamma(q) - std::lgamma(p + q));
  const double tiny = 1e-300;
  double f = 1.0, C = 1.0, D = 0.0;
  for (int j = 1; j <= 100000; ++j) {
    const int m = j / 2;
    const double dj = (j & 1) ? -(p + m) * (p + q + m) * x / ((p + 2 * m) * (p + 2 * m + 1))
                              : m * (q - m) * x / ((p + 2 * m - 1) * (p + 2 * m));
    D = 1.0 + dj * D;
    if (std::fabs(D) < tiny) D = tiny;
    D = 1.0 / D;
    C = 1.0 + dj / C;
    if (std::fabs(C) < tiny) C = tiny;
    const double delta = C * D;
    f *= delta;
    if (std::fabs(delta - 1.0) < 1e-16) break;
  }
  return std::exp(lnpre) / f;
}

struct SphereLaw {
  double q;     // (d - 1) / 2
  double lnB;   // ln B(1/2, q)
  explicit SphereLaw(int d) : q(0.5 * (d - 1)), lnB(std::lgamma(0.5) + std::lgamma(0.5 * (d - 1)) - std::lgamma(0.5 * d)) {}
  double tail(double x) const {  // P(u >= x), x >= 0
    if (x >= 1.0) return 0.0;
    return 0.5 * betainc_reg(q, 0.5, 1.0 - x * x);
  }
  double prob(double a, double b) const {  // P(a < u <= b)
    if (a >= 0.0) return tail(a) - tail(b);
    if (b <= 0.0) return tail(-b) - tail(-a);
    return 1.0 - tail(-a) - tail(b);
  }
  double g(double u) const {  // (1 - u^2)^q / (2 q B): int_a^b u f(u) du = g(a) - g(b)
    if (!(std::fabs(u) < 1.0)) return 0.0;
    return std::exp(q * std::log1p(-u * u) - std::log(2.0 * q) - lnB);
  }
};

}  // namespace

int tq_build_codebook(int32_t bits_mse, double sigma, tq_codebook *out) {
  if (!out || bits_mse < 1 || bits_mse > 3 || !(sigma > 0) || !std::isfinite(sigma))
    return TQ_ERR_INVALID_ARG;
  const int L = 1 << bits_mse;
  double c[TQ_MAX_LEVELS], t[TQ_MAX_LEVELS + 1];
  // start from an evenly spaced symmetric grid (N(0,1) units)
  for (int k = 0; k < L; ++k) c[k] = (2.0 * k - (L - 1)) / L * 2.0;
  int it = 0;
  bool done = false;
  for (it = 1; it <= 100000; ++it) {
    t[0] = -INFINITY;
    t[L] = INFINITY;
    for (int k = 1; k < L; ++k) t[k] = 0.5 * (c[k - 1] + c[k]);  // midpoint condition
    double delta = 0.0;
    for (int k = 0; k < L; ++k) {  // centroid condition: conditional mean of the cell
      double nc = (npdf(t[k]) - npdf(t[k + 1])) / cell_prob(t[k], t[k + 1]);
      delta = std::fmax(delta, std::fabs(nc - c[k]));
      c[k] = nc;
    }
    if (delta <= 1e-15) { done = true; break; }
  }
  if (!done) return TQ_ERR_NO_CONVERGENCE;
  double cs[TQ_MAX_LEVELS];
  for (int k = 0; k < L; ++k) cs[k] = 0.5 * (c[k] - c[L - 1 - k]);  // exact antisymmetry
  double mse = 1.0;
  t[0] = -INFINITY;
  t[L] = INFINITY;
  for (int k = 1; k < L; ++k) t[k] = 0.5 * (cs[k - 1] + cs[k]);
  for (int k = 0; k < L; ++k) mse -= cell_prob(t[k], t[k + 1]) * cs[k] * cs[k];
  for (int k = 0; k < L; ++k) cs[k] *= sigma;
  finish_codebook(bits_mse, sigma, cs, mse * sigma * sigma, it, out);
  return TQ_OK;
}

int tq_build_codebook_sphere(int32_t bits_mse, int32_t d, tq_codebook *out) {
  if (!out || bits_mse < 1 || bits_mse > 3 || d < 3) return TQ_ERR_INVALID_ARG;
  const int L = 1 << bits_mse;
  const SphereLaw law(d);
  const double sigma = 1.0 / std::sqrt(static_cast<double>(d));
  double c[TQ_MAX_LEVELS], t[TQ_MAX_LEVELS + 1];
  for (int k = 0; k < L; ++k) c[k] = std::fmax(-0.999, std::fmin(0.999, (2.0 * k - (L - 1)) / L * 2.0 * sigma));
  int it = 0;
  bool done = false;
  for (it = 1; it <= 100000; ++it) {
    t[0] = -1.0;
    t[L] = 1.0;
    for (int k = 1; k < L; ++k) t[k] = 0.5 * (c[k - 1] + c[k]);
    double delta = 0.0;
    for (int k = 0; k < L; ++k) {
      const double nc = (law.g(t[k]) - law.g(t[k + 1])) / law.prob(t[k], t[k + 1]);
      delta = std::fmax(delta, std::fabs(nc - c[k]));
      c[k] = nc;
    }
    if (delta <= 1e-13 * sigma) { done = true; break; }  // the beta CDF carries ~1e-15 relative rounding
  }
  if (!done) return TQ_ERR_NO_CONVERGENCE;
  double cs[TQ_MAX_LEVELS];
  for (int k = 0; k < L; ++k) cs[k] = 0.5 * (c[k] - c[L - 1 - k]);
  double mse = 1.0 / d;  // E[u^2]
  t[0] = -1.0;
  t[L] = 1.0;
  for (int k = 1; k < L; ++k) t[k] = 0.5 * (cs[k - 1] + cs[k]);
  for (int k = 0; k < L; ++k) mse -= law.prob(t[k], t[k + 1]) * cs[k] * cs[k];
  finish_codebook(bits_mse, sigma, cs, mse, it, out);
  return TQ_OK;
}

size_t tq_prepare_bytes(int32_t d, int32_t m) {
  if (m != d || !supported_d(d)) return 0;
  return tq::prep_layout(d, m).total;
}

int tq_prepare(const float *rot, const float *proj, int32_t d, int32_t m, void *blob) {
  if (!rot || !proj || !blob || d <= 0 || m != d) return TQ_ERR_INVALID_ARG;
  if (!supported_d(d)) return TQ_ERR_UNSUPPORTED;
  const tq::PrepLayout L = tq::prep_layout(d, m);
  auto *base = static_cast<unsigned char *>(blob);
  std::memset(base, 0, L.total);
  uint32_t hdr[4] = {tq::kPrepMagic, 1u, static_cast<uint32_t>(d), static_cast<uint32_t>(m)};
  std::memcpy(base, hdr, sizeof(hdr));
  auto *rotT = reinterpret_cast<float *>(base + L.rotT);
  auto *stT = reinterpret_cast<float *>(base + L.stT);
  auto *projT = reinterpret_cast<float *>(base + L.projT);
  auto *rot_hml = reinterpret_cast<uint16_t *>(base + L.rot_hml);
  auto *st_hml = reinterpret_cast<uint16_t *>(base + L.st_hml);
  auto *stnorm = reinterpret_cast<float *>(base + L.stnorm);
  const size_t dd = size_t(d) * d, md = size_t(m) * d;
  for (int j = 0; j < d; ++j)
    for (int k = 0; k < d; ++k) {
      rotT[size_t(k) * d + j] = rot[size_t(j) * d + k];
      split3(rot[size_t(j) * d + k], &rot_hml[size_t(j) * d + k], &rot_hml[dd + size_t(j) * d + k],
             &rot_hml[2 * dd + size_t(j) * d + k]);
    }
  for (int i = 0; i < m; ++i)
    for (int k = 0; k < d; ++k) projT[size_t(k) * m + i] = proj[size_t(i) * d + k];
  // S~ = S Pi^T in float64: S~[i][j] = sum_k S[i][k] Pi[j][k]
  std::vector<double> st(md);
  for (int i = 0; i < m; ++i)
    for (int j = 0; j < d; ++j) {
      double acc = 0.0;
      for (int k = 0; k < d; ++k) acc += double(proj[size_t(i) * d + k]) * double(rot[size_t(j) * d + k]);
      st[size_t(i) * d + j] = acc;
    }
  for (int i = 0; i < m; ++i) {
    double nrm = 0.0;
    for (int j = 0; j < d; ++j) {
      float f = static_cast<float>(st[size_t(i) * d + j]);
      stT[size_t(j) * m + i] = f;
      split3(f, &st_hml[size_t(i) * d + j], &st_hml[md + size_t(i) * d + j], &st_hml[2 * md + size_t(i) * d + j]);
      nrm += double(f) * double(f);
    }
    stnorm[i] = static_cast<float>(std::sqrt(nrm));
  }
  return TQ_OK;
}

int tq_quantize_kv(const tq_config *cfg, const void *k, const void *v, tq_dtype dt, int32_t batch,
                   int32_t n_new, const int64_t *dst_token, const tq_cache *kc, const tq_cache *vc,
                   uint32_t *status, float *dbg_scales, hipStream_t stream) {
  int e = check_config(cfg);
  if (e) return e;
  if (dt != TQ_F32 && dt != TQ_BF16) return TQ_ERR_INVALID_ARG;
  if (batch < 0 || n_new < 0) return TQ_ERR_INVALID_ARG;
  if (!k && !v) return TQ_ERR_INVALID_ARG;
  if (int64_t(batch) * n_new == 0) return TQ_OK;
  if (!dst_token) return TQ_ERR_INVALID_ARG;
  if ((status && (reinterpret_cast<uintptr_t>(status) & 3u)) || (dbg_scales && !aligned16(dbg_scales)))
    return TQ_ERR_INVALID_ARG;
  if ((k && !aligned16(k)) || (v && !aligned16(v)) || (reinterpret_cast<uintptr_t>(dst_token) & 7u))
    return TQ_ERR_INVALID_ARG;
  if (k && (e = check_cache(kc, cfg->k))) return e;
  if (v && (e = check_cache(vc, cfg->v))) return e;
  const tq::PrepLayout L = tq::prep_layout(cfg->d, cfg->m);
  const auto *prep = static_cast<const unsigned char *>(cfg->prep);
  const size_t per_tensor = size_t(batch) * cfg->n_kv_heads * n_new * 2;
  auto tensor_args = [&](int t) {
    const tq_cache *c = t ? vc : kc;
    const tq_tensor_spec &s = t ? cfg->v : cfg->k;
    tq::QuantTensorArgs ta{};
    ta.x = t ? v : k;
    ta.idx = c->idx;
    ta.sgn = c->sgn;
    ta.scl = c->scl;
    ta.cap = c->capacity;
    ta.layout = c->layout;
    ta.bq = s.bits_mse;
    ta.sketch = s.sketch;
    ta.cb = cb_f32(s.cb);
    ta.dbg = dbg_scales ? dbg_scales + t * per_tensor : nullptr;
    return ta;
  };
  auto fast_ok = [&](const tq::QuantTensorArgs &ta) {
    return (cfg->d == 128 || (cfg->d == 256 && dt == TQ_BF16)) && cb_symmetric(ta.cb);
  };
  tq::QuantArgs a{};
  a.dtype = dt;
  a.batch = batch;
  a.H = cfg->n_kv_heads;
  a.n_new = n_new;
  a.dst = dst_token;
  a.rotT = reinterpret_cast<const float *>(prep + L.rotT);
  a.stT = reinterpret_cast<const float *>(prep + L.stT);
  a.rot_hml = reinterpret_cast<const uint16_t *>(prep + L.rot_hml);
  a.st_hml = reinterpret_cast<const uint16_t *>(prep + L.st_hml);
  a.status = status;
  a.n_tensor = 1;
  if (k && v) {
    // K and V with one spec (bits, sketch, codebook) share one launch of the
    // d = 128 matrix-core kernel: its set-up (the matrices into registers) is paid
    // once.  (The d = 256 kernel streams its matrices and has no registers to spare
    // for a second tensor's arguments: one launch per tensor there.)
    const tq::QuantTensorArgs tk = tensor_args(0), tv = tensor_args(1);
    if (cfg->d == 128 && fast_ok(tk) && tk.bq == tv.bq && tk.sketch == tv.sketch &&
        std::memcmp(&tk.cb, &tv.cb, sizeof(tk.cb)) == 0) {
      a.t = tk;
      a.t2 = tv;
      a.n_tensor = 2;
      return tq::launch_quantize_fast(cfg->d, a, stream) != 0 ? TQ_ERR_LAUNCH : TQ_OK;
    }
  }
  for (int t = 0; t < 2; ++t) {
    if (!(t ? v : k)) continue;
    a.t = tensor_args(t);
    const int rc = fast_ok(a.t) ? tq::launch_quantize_fast(cfg->d, a, stream) : tq::launch_quantize(cfg->d, a, stream);
    if (rc != 0) return TQ_ERR_LAUNCH;
  }
  return TQ_OK;
}

size_t tq_decode_workspace_bytes(const tq_config *cfg, int32_t batch, int32_t max_len) {
  if (!cfg || batch < 0 || max_len < 0 || cfg->d <= 0 || cfg->m != cfg->d || cfg->n_kv_heads <= 0)
    return 0;
  return tq::decode_plan(*cfg, batch, max_len).total;
}

}  // extern "C"

namespace {

// Decode attention, dense (tau == 0) or Sparse V (0 < tau <= 1: a position's
// value is left out of the sum when its weight relative to the head's largest is
// below tau).
int decode_impl(const tq_config *cfg, const void *q, tq_dtype dt, int32_t batch, const int64_t *seq_start,
                const int32_t *seq_len, int32_t max_len, const tq_cache *kc, const tq_cache *vc, float sm_scale,
                float tau, float *out, uint32_t *status, void *workspace, size_t ws_bytes, hipStream_t stream) {
  int e = check_config(cfg);
  if (e) return e;
  if (dt != TQ_F32 && dt != TQ_BF16) return TQ_ERR_INVALID_ARG;
  if (batch < 0 || max_len < 0) return TQ_ERR_INVALID_ARG;
  if (batch == 0) return TQ_OK;
  if (!q || !seq_start || !seq_len || !out || !workspace) return TQ_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(out) || !aligned16(workspace)) return TQ_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(seq_start) & 7u) || (reinterpret_cast<uintptr_t>(seq_len) & 3u))
    return TQ_ERR_INVALID_ARG;
  if (status && (reinterpret_cast<uintptr_t>(status) & 3u)) return TQ_ERR_INVALID_ARG;
  if ((e = check_cache(kc, cfg->k)) || (e = check_cache(vc, cfg->v))) return e;
  if (kc->layout != TQ_LAYOUT_TOKEN_MAJOR || vc->layout != TQ_LAYOUT_BLOCK32) return TQ_ERR_UNSUPPORTED;
  if (!(sm_scale >= 0) || !std::isfinite(sm_scale)) return TQ_ERR_INVALID_ARG;
  if (!(tau >= 0.0f && tau <= 1.0f)) return TQ_ERR_INVALID_ARG;
  const int G = cfg->n_q_heads / cfg->n_kv_heads;
  if (G > 16) return TQ_ERR_UNSUPPORTED;
  const tq::DecodePlan p = tq::decode_plan(*cfg, batch, max_len);
  if (ws_bytes < p.total) return TQ_ERR_WORKSPACE;
  const tq::PrepLayout L = tq::prep_layout(cfg->d, cfg->m);
  const auto *prep = static_cast<const unsigned char *>(cfg->prep);
  auto *ws = static_cast<unsigned char *>(workspace);
  tq::DecodeArgs a{};
  for (int t = 0; t < 2; ++t) {
    const tq_cache *c = t ? vc : kc;
    const tq_tensor_spec &s = t ? cfg->v : cfg->k;
    tq::DecodeTensorArgs &ta = t ? a.v : a.k;
    ta.idx = c->idx;
    ta.sgn = c->sgn;
    ta.scl = c->scl;
    ta.cap = c->capacity;
    ta.bq = s.bits_mse;
    ta.sketch = s.sketch;
    ta.cb = cb_f32(s.cb);
  }
  a.q = q;
  a.dtype = dt;
  a.batch = batch;
  a.Hkv = cfg->n_kv_heads;
  a.Hq = cfg->n_q_heads;
  a.G = G;
  a.seq_start = seq_start;
  a.seq_len = seq_len;
  a.max_len = max_len;
  a.sm_scale = sm_scale > 0 ? sm_scale : static_cast<float>(1.0 / std::sqrt(double(cfg->d)));
  a.qbase = double(a.sm_scale) * 1.4426950408889634;  // log2(e): scores in base 2
  a.kv_fixed = -1;
  a.kappa = static_cast<float>(std::sqrt(M_PI / 2.0) / cfg->m);
  a.rot = cfg->rot;
  a.proj = cfg->proj;
  a.rotT = reinterpret_cast<const float *>(prep + L.rotT);
  a.projT = reinterpret_cast<const float *>(prep + L.projT);
  a.stnorm = reinterpret_cast<const float *>(prep + L.stnorm);
  a.qr = reinterpret_cast<float *>(ws + p.off_qr);
  a.qs = reinterpret_cast<float *>(ws + p.off_qs);
  a.part = reinterpret_cast<float *>(ws + p.off_part);
  a.split_tokens = p.split_tokens;
  a.n_split = p.n_split;
  a.qop = reinterpret_cast<uint32_t *>(ws + p.off_qop);
  a.qscale = ws + p.off_qscale;
  a.smax = reinterpret_cast<float *>(ws + p.off_smax);
  a.sparse_thr = tau > 0.0f ? std::log2(tau) : -INFINITY;
  for (int t = 0; t < 2; ++t) {
    const tq_codebook &cb = t ? cfg->v.cb : cfg->k.cb;
    double *wc = t ? a.walsh_v : a.walsh_k;
    wc[0] = cb.walsh[1];
    wc[1] = cb.levels > 2 ? cb.walsh[2] : 0.0;
    wc[2] = cb.levels > 4 ? cb.walsh[4] : 0.0;
    wc[3] = cb.levels > 4 ? cb.walsh[7] : 0.0;
  }
  a.out = out;
  a.status = status;
  // the matrix-core decode expands the codebook over odd Walsh terms only, which
  // holds for an antisymmetric codebook (every Lloyd-Max codebook of a symmetric law)
  const bool fast = p.fast && cb_symmetric(a.k.cb) && cb_symmetric(a.v.cb);
  const bool sparse = tau > 0.0f;
  if (sparse && !fast) return TQ_ERR_UNSUPPORTED;  // Sparse V runs on the matrix-core kernels only
  const int rc = fast ? tq::launch_decode_fast(cfg->d, p.rb, a, stream, sparse) : tq::launch_decode(cfg->d, a, stream);
  if (rc != 0) return TQ_ERR_LAUNCH;
  return TQ_OK;
}

}  // namespace

extern "C" {

int tq_decode_attention(const tq_config *cfg, const void *q, tq_dtype dt, int32_t batch,
                        const int64_t *seq_start, const int32_t *seq_len, int32_t max_len,
                        const tq_cache *kc, const tq_cache *vc, float sm_scale, float *out,
                        uint32_t *status, void *workspace, size_t ws_bytes, hipStream_t stream) {
  return decode_impl(cfg, q, dt, batch, seq_start, seq_len, max_len, kc, vc, sm_scale, 0.0f, out, status,
                     workspace, ws_bytes, stream);
}

int tq_decode_attention_sparse_v(const tq_config *cfg, const void *q, tq_dtype dt, int32_t batch,
                                 const int64_t *seq_start, const int32_t *seq_len, int32_t max_len,
                                 const tq_cache *kc, const tq_cache *vc, float sm_scale, float tau, float *out,
                                 uint32_t *status, void *workspace, size_t ws_bytes, hipStream_t stream) {
  return decode_impl(cfg, q, dt, batch, seq_start, seq_len, max_len, kc, vc, sm_scale, tau, out, status,
                     workspace, ws_bytes, stream);
}

namespace {

// Queries per split-pass block of tq_score_keys: 16 at d = 128 when n_q allows
// (four MFMA row blocks, whose operands fit in registers there), else 8.
int32_t score_group(const tq_config &cfg, int32_t n_q) { return cfg.d == 128 && n_q % 16 == 0 ? 16 : 8; }

// Workspace of tq_score_keys: the query operands and constants of n_q queries,
// and 64 words that scoring lanes outside the key range write instead.
struct ScorePlan {
  int32_t group, split_tokens, n_split;
  size_t off_qop, off_qscale, off_dummy, total;
};

ScorePlan score_plan(const tq_config &cfg, int32_t n_q, int32_t max_n) {
  ScorePlan p{};
  p.group = score_group(cfg, n_q);
  const int64_t groups = n_q / p.group;
  int64_t st = groups > 0 ? (int64_t(max_n) * groups + 511) / 512 : 256;  // about 512 work-groups
  st = (st + 255) / 256 * 256;
  if (st > 1024) st = 1024;
  if (st < 256) st = 256;
  p.split_tokens = static_cast<int32_t>(st);
  p.n_split = static_cast<int32_t>((int64_t(max_n) + 63 + st - 1) / st);
  if (p.n_split < 1) p.n_split = 1;
  size_t o = 0;
  p.off_qop = o;    o = tq::align256(o + size_t(groups) * tq::q_operand_bytes(cfg.d, p.group));
  p.off_qscale = o; o = tq::align256(o + size_t(groups) * tq::q_scale_bytes());
  p.off_dummy = o;  o = tq::align256(o + 64 * 4);
  p.total = o;
  return p;
}

}  // namespace

size_t tq_score_workspace_bytes(const tq_config *cfg, int32_t n_q, int32_t max_n) {
  if (!cfg || n_q <= 0 || n_q % 8 || max_n < 0 || cfg->d <= 0) return 0;
  return score_plan(*cfg, n_q, max_n).total;
}

int tq_score_keys(const tq_config *cfg, const void *q, tq_dtype dt, int32_t n_q, const tq_cache *kc,
                  int32_t kv_head, int64_t start, int32_t n, float *scores, uint32_t *status,
                  void *workspace, size_t ws_bytes, hipStream_t stream) {
  int e = check_config(cfg);
  if (e) return e;
  if (dt != TQ_F32 && dt != TQ_BF16) return TQ_ERR_INVALID_ARG;
  if (n_q <= 0 || n_q % 8 || n < 0 || start < 0) return TQ_ERR_INVALID_ARG;
  if (kv_head < 0 || kv_head >= cfg->n_kv_heads) return TQ_ERR_INVALID_ARG;
  if (n == 0) return TQ_OK;
  if (!q || !scores || !workspace) return TQ_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(workspace) || (reinterpret_cast<uintptr_t>(scores) & 3u))
    return TQ_ERR_INVALID_ARG;
  if (status && (reinterpret_cast<uintptr_t>(status) & 3u)) return TQ_ERR_INVALID_ARG;
  if ((e = check_cache(kc, cfg->k))) return e;
  if (kc->layout != TQ_LAYOUT_TOKEN_MAJOR) return TQ_ERR_UNSUPPORTED;
  if (start + n > kc->capacity) return TQ_ERR_INVALID_ARG;
  if (cfg->d != 128 && cfg->d != 256) return TQ_ERR_UNSUPPORTED;
  const ScorePlan p = score_plan(*cfg, n_q, n);
  if (ws_bytes < p.total) return TQ_ERR_WORKSPACE;
  const tq::PrepLayout L = tq::prep_layout(cfg->d, cfg->m);
  const auto *prep = static_cast<const unsigned char *>(cfg->prep);
  auto *ws = static_cast<unsigned char *>(workspace);
  tq::DecodeArgs a{};
  a.k.idx = kc->idx;
  a.k.sgn = kc->sgn;
  a.k.scl = kc->scl;
  a.k.cap = kc->capacity;
  a.k.bq = cfg->k.bits_mse;
  a.k.sketch = cfg->k.sketch;
  a.k.cb = cb_f32(cfg->k.cb);
  if (!cb_symmetric(a.k.cb)) return TQ_ERR_UNSUPPORTED;
  const tq_codebook &cb = cfg->k.cb;
  a.walsh_k[0] = cb.walsh[1];
  a.walsh_k[1] = cb.levels > 2 ? cb.walsh[2] : 0.0;
  a.walsh_k[2] = cb.levels > 4 ? cb.walsh[4] : 0.0;
  a.walsh_k[3] = cb.levels > 4 ? cb.walsh[7] : 0.0;
  a.q = q;
  a.dtype = dt;
  a.batch = 1;
  a.Hq = n_q;
  a.G = p.group;
  a.Hkv = n_q / p.group;  // query groups; every one reads key head kv_head
  a.kv_fixed = kv_head;
  a.seq_start = nullptr;
  a.seq_len = nullptr;
  a.fix_start = start;
  a.fix_len = n;
  a.max_len = n;
  a.sm_scale = 1.0f;
  a.qbase = 1.0;  // raw inner products
  a.kappa = static_cast<float>(std::sqrt(M_PI / 2.0) / cfg->m);
  a.rotT = reinterpret_cast<const float *>(prep + L.rotT);
  a.projT = reinterpret_cast<const float *>(prep + L.projT);
  a.stnorm = reinterpret_cast<const float *>(prep + L.stnorm);
  a.split_tokens = p.split_tokens;
  a.n_split = p.n_split;
  a.qop = reinterpret_cast<uint32_t *>(ws + p.off_qop);
  a.qscale = ws + p.off_qscale;
  a.scores = scores;
  a.score_ld = n;
  a.score_dummy = reinterpret_cast<float *>(ws + p.off_dummy);
  a.status = status;
  if (tq::launch_score_fast(cfg->d, a, stream) != 0) return TQ_ERR_LAUNCH;
  return TQ_OK;
}

}  // extern "C"
