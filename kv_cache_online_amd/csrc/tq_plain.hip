// Reference-grade HIP kernels for gfx950: quantize and decode over the packed
// cache, written for clarity and exactness (float64 accumulation on the
// vector ALU, which is full rate on CDNA).  They define the device-side
// semantics that the fast kernels must reproduce.
//
// Method: ast-softpro.ru, "Технология TurboQuant и её применение с локальными
// LLM", section 1.2 "Как работает TurboQuant" -- stage 1 rotation by Pi and a
// per-coordinate Lloyd-Max cell; stage 2 sign(S r) of the residual and ||r||_2.
// The residual is formed in the rotated frame, rho_vec = Pi x - nu16 c[idx],
// and its sketch as S~ rho_vec with S~ = S Pi^T precomputed on the host; both
// equal the original-space quantities r and S r because Pi is orthogonal.

#include <hip/hip_runtime.h>

#include <cmath>

#include "tq_common.h"
#include "tq_device.h"

namespace tq {
namespace {

// ------------------------------------------------------------------ quantize --
// One wavefront per vector; 4 vectors per 256-thread block.  Lane l owns
// coordinates / sketch rows l, l + 64, ...
template <int D>
__global__ __launch_bounds__(256) void quantize_plain(QuantArgs a) {
  constexpr int R = D / kWave;
  __shared__ float xs[4][D];
  __shared__ float rs[4][D];
  __shared__ float cen[TQ_MAX_LEVELS];
  __shared__ float thr[TQ_MAX_LEVELS - 1];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  if (threadIdx.x < TQ_MAX_LEVELS) cen[threadIdx.x] = a.t.cb.cen[threadIdx.x];
  if (threadIdx.x < TQ_MAX_LEVELS - 1) thr[threadIdx.x] = a.t.cb.thr[threadIdx.x];
  const int64_t n_vec = int64_t(a.batch) * a.H * a.n_new;
  const int64_t vid = int64_t(blockIdx.x) * 4 + wave;
  const bool active = vid < n_vec;
  const int64_t vv = active ? vid : 0;
  const int t = static_cast<int>(vv % a.n_new);
  const int h = static_cast<int>((vv / a.n_new) % a.H);
  const int b = static_cast<int>(vv / (int64_t(a.n_new) * a.H));
  const int L = a.t.cb.levels;

  // stage 1: load, norm ||x|| (float64), rotation z = Pi x
  double ss = 0.0;
  bool finite = true;
  for (int r = 0; r < R; ++r) {
    const int j = lane + kWave * r;
    float xv = active ? load_in(a.t.x, a.dtype, size_t(vv) * D + j) : 0.0f;
    finite &= isfinite(xv);
    xs[wave][j] = xv;
    ss += double(xv) * double(xv);
  }
  __syncthreads();
  const double nu = sqrt(wave_sum_d(ss));
  const bool any_bad = __ballot(!finite) != 0;
  bool over = false;
  const uint32_t nu_bits = f16_bits(nu, &over);
  const float nu16 = f16_val(nu_bits);
  const float nuf = static_cast<float>(nu);

  int code[R];
  double rr = 0.0;
  for (int r = 0; r < R; ++r) {
    const int j = lane + kWave * r;
    double z = 0.0;
    for (int k = 0; k < D; ++k) z = fma(double(a.rotT[size_t(k) * D + j]), double(xs[wave][k]), z);
    const float u = nu > 0.0 ? static_cast<float>(z / nu) : 0.0f;
    int c = 0;
    for (int q = 0; q < L - 1; ++q) c += (u >= thr[q]);
    if (!(nu > 0.0)) c = L / 2;
    code[r] = c;
    const double rho_j = z - double(nu16) * double(cen[c]);  // rotated-frame residual
    rs[wave][j] = static_cast<float>(rho_j);
    rr += rho_j * rho_j;
  }
  (void)nuf;
  __syncthreads();
  const double rho = a.t.sketch ? sqrt(wave_sum_d(rr)) : 0.0;
  uint32_t rho_bits = 0;
  if (a.t.sketch) rho_bits = f16_bits(rho, &over);

  // stage 2: sign sketch p = S~ rho_vec
  bool sgn[R];
  if (a.t.sketch) {
    for (int r = 0; r < R; ++r) {
      const int i = lane + kWave * r;
      double p = 0.0;
      for (int j = 0; j < D; ++j) p = fma(double(a.stT[size_t(j) * D + i]), double(rs[wave][j]), p);
      sgn[r] = p >= 0.0;
    }
  }
  if (!active) return;
  if (a.status && lane == 0) {
    uint32_t f = (any_bad ? TQ_FLAG_NONFINITE_INPUT : 0u) | (over ? TQ_FLAG_SCALE_OVERFLOW : 0u);
    if (f) atomicOr(a.status, f);
  }
  if (a.t.dbg && lane == 0) {
    a.t.dbg[vv * 2 + 0] = static_cast<float>(nu);
    a.t.dbg[vv * 2 + 1] = static_cast<float>(rho);
  }
  const int64_t slot = a.dst[b] + t;
  if (slot < 0 || slot >= a.t.cap) {
    if (a.status && lane == 0) atomicOr(a.status, TQ_FLAG_OUT_OF_RANGE);
    return;
  }
  const int64_t hs = int64_t(h) * a.t.cap + slot;
  if (lane == 0) {
    a.t.scl[hs * 2 + 0] = static_cast<uint16_t>(nu_bits);
    a.t.scl[hs * 2 + 1] = static_cast<uint16_t>(rho_bits);
  }
  if (a.t.layout == TQ_LAYOUT_TOKEN_MAJOR) {
    constexpr int W = D / 32;
    for (int q = 0; q < a.t.bq; ++q)
      for (int r = 0; r < R; ++r) {
        const uint64_t m = __ballot((code[r] >> q) & 1);
        if (lane < 2) a.t.idx[(hs * a.t.bq + q) * W + 2 * r + lane] = static_cast<uint32_t>(m >> (32 * lane));
      }
    if (a.t.sketch)
      for (int r = 0; r < R; ++r) {
        const uint64_t m = __ballot(sgn[r]);
        if (lane < 2) a.t.sgn[hs * W + 2 * r + lane] = static_cast<uint32_t>(m >> (32 * lane));
      }
  } else {  // BLOCK32: one bit per (plane, coordinate) word of the 32-slot block
    const int64_t blk = int64_t(h) * (a.t.cap / 32) + (slot >> 5);
    const uint32_t bit = 1u << (slot & 31);
    for (int q = 0; q < a.t.bq; ++q)
      for (int r = 0; r < R; ++r) {
        uint32_t *w = &a.t.idx[(blk * a.t.bq + q) * D + lane + kWave * r];
        if ((code[r] >> q) & 1) atomicOr(w, bit);
        else atomicAnd(w, ~bit);
      }
    if (a.t.sketch)
      for (int r = 0; r < R; ++r) {
        uint32_t *w = &a.t.sgn[blk * D + lane + kWave * r];
        if (sgn[r]) atomicOr(w, bit);
        else atomicAnd(w, ~bit);
      }
  }
}

// -------------------------------------------------------------------- decode --
// Query prep: q_rot = Pi q and q_s = S q per (sequence, query head).
template <int D>
__global__ __launch_bounds__(256) void decode_qprep_plain(DecodeArgs a) {
  __shared__ float qv[D];
  const int64_t bh = blockIdx.x;
  for (int j = threadIdx.x; j < D; j += blockDim.x) qv[j] = load_in(a.q, a.dtype, size_t(bh) * D + j);
  __syncthreads();
  for (int j = threadIdx.x; j < D; j += blockDim.x) {
    double zr = 0.0, zs = 0.0;
    for (int k = 0; k < D; ++k) {
      zr = fma(double(a.rotT[size_t(k) * D + j]), double(qv[k]), zr);
      zs = fma(double(a.projT[size_t(k) * D + j]), double(qv[k]), zs);
    }
    a.qr[size_t(bh) * D + j] = static_cast<float>(zr);
    a.qs[size_t(bh) * D + j] = static_cast<float>(zs);
  }
}

__device__ inline void clip_range(const DecodeArgs &a, int b, int64_t *start, int64_t *len) {
  int64_t s = a.seq_start[b], n = a.seq_len[b];
  const int64_t cap = a.k.cap < a.v.cap ? a.k.cap : a.v.cap;
  bool bad = false;
  if (n < 0) { n = 0; bad = true; }
  if (s < 0 || s > cap) { s = 0; n = 0; bad = true; }
  if (s + n > cap) { n = cap - s; bad = true; }
  if (n > a.max_len) { n = a.max_len; bad = true; }  // the launch covers max_len slots
  if (bad && a.status && threadIdx.x == 0 && blockIdx.x == 0 && blockIdx.y == 0) atomicOr(a.status, TQ_FLAG_OUT_OF_RANGE);
  *start = s;
  *len = n;
}

// Split partials: one wavefront per (split, kv head, sequence).  Scores with
// one lane per token, online softmax per query head, then value accumulation
// with one lane per coordinate.  Output per query head: running max m, sum l,
// A = sum_t p_t nu16_t c[idx_t] (rotated frame), B = sum_t p_t rho16_t (2 sgn_t - 1).
// GM is a power of two >= G = a.G (the group size need not be one).
template <int D, int GM>
__global__ __launch_bounds__(64) void decode_partial_plain(DecodeArgs a) {
  constexpr int R = D / kWave, W = D / 32;
  const int G = a.G;
  __shared__ float qr[GM][D], qs[GM][D];
  __shared__ float ck[TQ_MAX_LEVELS], cv[TQ_MAX_LEVELS];
  __shared__ float P[GM][kWave];
  __shared__ float vnu[kWave], vrho[kWave];
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
  int64_t start, len;
  clip_range(a, b, &start, &len);
  if (lane < TQ_MAX_LEVELS) {
    ck[lane] = a.k.cb.cen[lane];
    cv[lane] = a.v.cb.cen[lane];
  }
  for (int g = 0; g < GM; ++g)
    for (int r = 0; r < R; ++r) {
      const size_t o = (size_t(b) * a.Hq + size_t(h) * G + g) * D + lane + kWave * r;
      qr[g][lane + kWave * r] = g < G ? a.qr[o] : 0.0f;
      qs[g][lane + kWave * r] = g < G ? a.qs[o] : 0.0f;
    }
  __syncthreads();
  float m[GM], l[GM], A[GM][R], B[GM][R];
  for (int g = 0; g < GM; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.0f;
    for (int r = 0; r < R; ++r) A[g][r] = B[g][r] = 0.0f;
  }
  const int64_t t0 = int64_t(split) * a.split_tokens;
  const int64_t t1 = t0 + a.split_tokens < len ? t0 + a.split_tokens : len;
  const int64_t kcap = a.k.cap, vcap = a.v.cap;
  for (int64_t tb = t0; tb < t1; tb += kWave) {
    const int64_t t = tb + lane;
    const bool valid = t < t1;
    const int64_t slot = start + (valid ? t : tb);
    float s[GM];
    {
      uint32_t kw[3][W], sw[W];
      const int64_t hs = int64_t(h) * kcap + slot;
      for (int q = 0; q < 3; ++q)
        for (int w = 0; w < W; ++w) kw[q][w] = q < a.k.bq ? a.k.idx[(hs * a.k.bq + q) * W + w] : 0u;
      for (int w = 0; w < W; ++w) sw[w] = a.k.sketch ? a.k.sgn[hs * W + w] : 0u;
      const float knu = f16_val(a.k.scl[hs * 2]), krho = f16_val(a.k.scl[hs * 2 + 1]);
      for (int g = 0; g < GM; ++g) {
        float sd = 0.0f, sg = 0.0f;
        for (int j = 0; j < D; ++j) {
          const int w = j >> 5, bt = j & 31;
          const int c = ((kw[0][w] >> bt) & 1) | (((kw[1][w] >> bt) & 1) << 1) | (((kw[2][w] >> bt) & 1) << 2);
          sd = fmaf(qr[g][j], ck[c], sd);
          sg += ((sw[w] >> bt) & 1) ? qs[g][j] : -qs[g][j];
        }
        const float sc = a.k.sketch ? fmaf(a.kappa * krho, sg, knu * sd) : knu * sd;
        s[g] = valid ? a.sm_scale * sc : -INFINITY;
      }
      const int64_t hv = int64_t(h) * vcap + slot;
      vnu[lane] = valid ? f16_val(a.v.scl[hv * 2]) : 0.0f;
      vrho[lane] = valid ? f16_val(a.v.scl[hv * 2 + 1]) : 0.0f;
    }
    for (int g = 0; g < GM; ++g) {
      const float tmax = wave_max_f(s[g]);
      const float mn = fmaxf(m[g], tmax);
      const float alpha = m[g] == -INFINITY ? 0.0f : expf(m[g] - mn);
      const float p = valid ? expf(s[g] - mn) : 0.0f;
      l[g] = l[g] * alpha + wave_sum_f(p);
      m[g] = mn;
      P[g][lane] = p;
      for (int r = 0; r < R; ++r) {
        A[g][r] *= alpha;
        B[g][r] *= alpha;
      }
    }
    __syncthreads();
    // values: lane owns coordinates lane + 64 r; walk the 32-slot blocks of this tile
    const int64_t s0 = start + tb, s1 = start + (tb + kWave < t1 ? tb + kWave : t1);
    for (int64_t blk = s0 >> 5; blk <= (s1 - 1) >> 5; ++blk) {
      uint32_t vw[3][R], vs[R];
      const int64_t hb = int64_t(h) * (vcap / 32) + blk;
      for (int q = 0; q < 3; ++q)
        for (int r = 0; r < R; ++r) vw[q][r] = q < a.v.bq ? a.v.idx[(hb * a.v.bq + q) * D + lane + kWave * r] : 0u;
      for (int r = 0; r < R; ++r) vs[r] = a.v.sketch ? a.v.sgn[hb * D + lane + kWave * r] : 0u;
      const int64_t lo = (blk << 5) > s0 ? (blk << 5) : s0;
      const int64_t hi = ((blk + 1) << 5) < s1 ? ((blk + 1) << 5) : s1;
      for (int64_t sl = lo; sl < hi; ++sl) {
        const int tt = static_cast<int>(sl - s0), bt = static_cast<int>(sl & 31);
        for (int r = 0; r < R; ++r) {
          const int c = ((vw[0][r] >> bt) & 1) | (((vw[1][r] >> bt) & 1) << 1) | (((vw[2][r] >> bt) & 1) << 2);
          const float cvv = cv[c] * vnu[tt];
          const float sgv = ((vs[r] >> bt) & 1) ? vrho[tt] : -vrho[tt];
          for (int g = 0; g < GM; ++g) {
            A[g][r] = fmaf(P[g][tt], cvv, A[g][r]);
            B[g][r] = fmaf(P[g][tt], sgv, B[g][r]);
          }
        }
      }
    }
    __syncthreads();
  }
  const int stride = 2 + 2 * D;
  for (int g = 0; g < G; ++g) {
    float *o = a.part + ((size_t(b) * a.Hq + size_t(h) * G + g) * a.n_split + split) * stride;
    if (lane == 0) {
      o[0] = m[g];
      o[1] = l[g];
    }
    for (int r = 0; r < R; ++r) {
      o[2 + lane + kWave * r] = A[g][r];
      o[2 + D + lane + kWave * r] = a.v.sketch ? B[g][r] : 0.0f;
    }
  }
}

// Log-sum-exp merge of the split partials, then out = (Pi^T A + kappa S^T B) / l.
template <int D>
__global__ __launch_bounds__(256) void decode_merge_plain(DecodeArgs a) {
  __shared__ float As[D], Bs[D];
  __shared__ float lsum;
  const int64_t bh = blockIdx.x;
  const int stride = 2 + 2 * D;
  const float *base = a.part + size_t(bh) * a.n_split * stride;
  float M = -INFINITY;
  for (int s = 0; s < a.n_split; ++s)
    if (base[size_t(s) * stride + 1] > 0.0f) M = fmaxf(M, base[size_t(s) * stride]);
  for (int j = threadIdx.x; j < D; j += blockDim.x) {
    float aj = 0.0f, bj = 0.0f, lj = 0.0f;
    for (int s = 0; s < a.n_split; ++s) {
      const float *p = base + size_t(s) * stride;
      if (!(p[1] > 0.0f)) continue;
      const float w = expf(p[0] - M);
      aj = fmaf(w, p[2 + j], aj);
      bj = fmaf(w, p[2 + D + j], bj);
      lj = fmaf(w, p[1], lj);
    }
    As[j] = aj;
    Bs[j] = bj;
    if (j == 0) lsum = lj;
  }
  __syncthreads();
  for (int j = threadIdx.x; j < D; j += blockDim.x) {
    float o = 0.0f;
    if (lsum > 0.0f) {
      double acc = 0.0;
      for (int k = 0; k < D; ++k) acc = fma(double(a.rot[size_t(k) * D + j]), double(As[k]), acc);
      if (a.v.sketch) {
        double sb = 0.0;
        for (int i = 0; i < D; ++i) sb = fma(double(a.proj[size_t(i) * D + j]), double(Bs[i]), sb);
        acc += double(a.kappa) * sb;
      }
      o = static_cast<float>(acc / double(lsum));
    }
    a.out[size_t(bh) * D + j] = o;
  }
}

template <int D>
int launch_quantize_d(const QuantArgs &a, hipStream_t s) {
  const int64_t n = int64_t(a.batch) * a.H * a.n_new;
  const unsigned grid = static_cast<unsigned>((n + 3) / 4);
  hipLaunchKernelGGL(quantize_plain<D>, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError() != hipSuccess;
}

template <int D, int GM>
int launch_partial(const DecodeArgs &a, hipStream_t s) {
  hipLaunchKernelGGL((decode_partial_plain<D, GM>), dim3(a.n_split, a.Hkv, a.batch), dim3(64), 0, s, a);
  return 0;
}

template <int D>
int launch_decode_d(const DecodeArgs &a, hipStream_t s) {
  const unsigned nq = static_cast<unsigned>(a.batch * a.Hq);
  hipLaunchKernelGGL(decode_qprep_plain<D>, dim3(nq), dim3(256), 0, s, a);
  // the kernel's head loops run to the next power of two; heads past G are idle
  if (a.G < 1 || a.G > 16) return 1;
  if (a.G == 1) launch_partial<D, 1>(a, s);
  else if (a.G == 2) launch_partial<D, 2>(a, s);
  else if (a.G <= 4) launch_partial<D, 4>(a, s);
  else if (a.G <= 8) launch_partial<D, 8>(a, s);
  else launch_partial<D, 16>(a, s);
  hipLaunchKernelGGL(decode_merge_plain<D>, dim3(nq), dim3(256), 0, s, a);
  return hipGetLastError() != hipSuccess;
}

}  // namespace

int launch_quantize(int d, const QuantArgs &a, hipStream_t s) {
  switch (d) {
    case 64: return launch_quantize_d<64>(a, s);
    case 128: return launch_quantize_d<128>(a, s);
    case 256: return launch_quantize_d<256>(a, s);
    default: return 1;
  }
}

int launch_decode(int d, const DecodeArgs &a, hipStream_t s) {
  switch (d) {
    case 64: return launch_decode_d<64>(a, s);
    case 128: return launch_decode_d<128>(a, s);
    case 256: return launch_decode_d<256>(a, s);
    default: return 1;
  }
}

}  // namespace tq
