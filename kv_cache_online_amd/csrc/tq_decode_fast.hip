// Decode attention over the packed caches on the CDNA4 matrix cores.
//
// The speed of decode over a compressed cache comes from moving fewer bytes
// (ast-softpro.ru, "Технология TurboQuant и её применение с локальными LLM",
// section 1.3).  On MI355X the vector ALU cannot keep up with HBM if every
// query head takes its own dot products with every unpacked coordinate, so the
// contractions of all G query heads of a kv head run as exact integer MFMAs
// (v_mfma_i32_16x16x64_i8):
//
//  * Bit-plane operands.  A codebook value is an odd function of the +-1
//    bit-planes of its index (Walsh expansion: b' = 1, 2 are linear, b' = 3 adds
//    the triple product s0 s1 s2 = 2 (b0 ^ b1 ^ b2) - 1).  With s = 2 b - 1 a
//    dot product with a plane is 2 <v, b> - sum(v), so the MFMA only needs 0/1
//    bits.  A packed word (shifted right by 4 for the odd nibbles) ANDed with
//    0x01010101 << k yields four int8 operand bytes bit << k, k = 0..3; the
//    other operand is pre-divided by 2^k.
//  * Fixed-point slices.  Each real operand v (Walsh-weighted rotated query,
//    sketched query, softmax weight times scale) becomes F = rint(v 2^E) with
//    |F| < 2^30, written as four signed base-256 digits (bytes of
//    (F + 0x808080) ^ 0x808080).  Rows of the MFMA are (query head, digit), so
//    16 rows hold 4 heads; G = 8 uses two row blocks.  Digit sums are recombined
//    exactly in float64.
//  * Exact split maximum.  Scores of a split (at most 8192 / G slots) are kept in
//    LDS; the value pass runs after the split's maximum is known, so the integer
//    accumulators never need rescaling.
//
// Keys are read token-major (a token's planes contiguous: the score contraction
// runs over coordinates); values in the 32-slot transposed layout (a word holds
// one coordinate of 32 consecutive slots: the value contraction runs over
// tokens).  Splits are aligned to absolute 64-slot tiles.

#include <hip/hip_runtime.h>

#include <cmath>

#include "tq_common.h"
#include "tq_device.h"

namespace tq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kSigPlane = 4;     // operand / accumulator slot of the sign plane

__device__ inline int n_walsh(int bq) { return bq == 3 ? 4 : bq; }

__device__ inline float load_q(const void *x, int dtype, size_t i) {
  if (dtype == TQ_BF16) return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t *>(x)[i]) << 16);
  return static_cast<const float *>(x)[i];
}

__device__ inline float f16v(uint32_t bits) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits & 0xFFFFu)));
}

__device__ inline v4i expand(uint32_t w, uint32_t sh, const uint32_t (&m)[4]) {
  w >>= sh;
  v4i r;
  r.x = static_cast<int>(w & m[0]);
  r.y = static_cast<int>(w & m[1]);
  r.z = static_cast<int>(w & m[2]);
  r.w = static_cast<int>(w & m[3]);
  return r;
}

// Word of Walsh plane p (p < 3: index bit-plane p; p == 3: b0 ^ b1 ^ b2, whose
// +-1 form is the triple product s0 s1 s2).
template <int PM>
__device__ inline uint32_t plane_word(int p, uint32_t w0, uint32_t w1, uint32_t w2) {
  return p == 0 ? w0 : p == 1 ? w1 : p == 2 ? w2 : (w0 ^ w1 ^ w2);
}

__device__ inline v4i mfma(v4i a, v4i b, v4i c) { return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0); }

// sum_l 256^l c_l, exact: every digit sum is below 2^21 in magnitude (operand
// bytes <= 8, digits <= 128, at most 2048 terms), so pairs combine in int32.
__device__ inline double combine(v4i c) {
  const int32_t lo = c.x + (c.y << 8), hi = c.z + (c.w << 8);
  return fma(static_cast<double>(hi), 65536.0, static_cast<double>(lo));
}

// The +-1 form sum_t w_t (2 b_t - 1) from digit sums x of weight x bit and k of
// weight x 1: 2 x_l - k_l per digit (each below 2^23), then recombined.
__device__ inline double pm_form(v4i x, v4i k) {
  const v4i r = {2 * x.x - k.x, 2 * x.y - k.y, 2 * x.z - k.z, 2 * x.w - k.w};
  const int32_t lo = r.x + (r.y << 8), hi = r.z + (r.w << 8);
  return fma(static_cast<double>(hi), 65536.0, static_cast<double>(lo));
}

__device__ inline uint32_t digits(int32_t f) { return static_cast<uint32_t>(f + 0x00808080) ^ 0x00808080u; }

// Exponent E with vmax * 2^E < 2^30 (0 for vmax == 0).
__device__ inline int fix_exp(double vmax) { return vmax > 0.0 ? 29 - ilogb(vmax) : 0; }

__device__ inline void clip_seq(const DecodeArgs &a, int b, int64_t *start, int64_t *len) {
  const bool fixed = a.seq_start == nullptr;  // key scoring: one slot range, keys only
  int64_t s = fixed ? a.fix_start : a.seq_start[b], n = fixed ? a.fix_len : a.seq_len[b];
  const int64_t cap = fixed ? a.k.cap : a.k.cap < a.v.cap ? a.k.cap : a.v.cap;
  bool bad = false;
  if (n < 0) { n = 0; bad = true; }
  if (s < 0 || s > cap) { s = 0; n = 0; bad = true; }
  if (s + n > cap) { n = cap - s; bad = true; }
  if (bad && a.status && threadIdx.x == 0 && blockIdx.x == 0 && blockIdx.y == 0) atomicOr(a.status, TQ_FLAG_OUT_OF_RANGE);
  *start = s;
  *len = n;
}

// ------------------------------------------------------------- query prep ---
// Block (sequence, query head, slice t) of 2 d / 64: slice t < d / 64 covers
// coordinates 64 t .. 64 t + 63 of q_rot = Pi q (the Walsh planes' operands),
// slice t >= d / 64 the same coordinates of q_s = S q (the sign plane's).  It
// computes its 64 products in fp32 (about 2^-24 relative error, far inside what
// the scores need) from the transposed matrices, so that a wave's loads are
// contiguous, and writes this head's four rows (one per digit) of its operand
// entries.  The fixed-point exponent of a plane must be the same in every
// slice, so it comes from a bound every slice can compute: |(Pi q)_j| <= ||q||
// (Pi is orthogonal) and |(S q)_i| <= max_i ||S_i|| ||q|| (the row norms of
// S~ = S Pi^T, equal to those of S), with 2^-10 to spare for rounding.  The
// exact corrections sum_j F_j 2^shift_j are summed by the split pass.
template <int D>
__global__ __launch_bounds__(256) void decode_qprep_fast(DecodeArgs a) {
  constexpr int C = D / 64, NSL = 2 * D / 64, KPT = D / 4;
  __shared__ float q[D];
  __shared__ float part[4][64];
  __shared__ float vals[64];
  __shared__ float red[2][4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bh = blockIdx.x / NSL, t = blockIdx.x % NSL;
  const int b = bh / a.Hq, hq = bh % a.Hq;
  const int kvh = hq / a.G, hl = hq % a.G, rb = hl >> 2, row0 = (hl & 3) * 4;
  const int RB = a.G / 4;
  const bool sgn = t >= D / 64;
  if (sgn && !a.k.sketch) return;  // no sign plane
  const int c0 = (sgn ? t - D / 64 : t) * 64;
  // column c0 + lane of Pi^T or S^T, rows wave KPT .. wave KPT + KPT - 1
  const float *mt = (sgn ? a.projT : a.rotT) + c0 + lane + size_t(wave) * KPT * D;
  float m[KPT];
#pragma unroll
  for (int i = 0; i < KPT; ++i) m[i] = mt[size_t(i) * D];
  float ss = 0.0f, smax = 0.0f;
  for (int j = tid; j < D; j += 256) {
    const float v = load_q(a.q, a.dtype, size_t(bh) * D + j);
    q[j] = v;
    ss = fmaf(v, v, ss);
    if (sgn) smax = fmaxf(smax, a.stnorm[j]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    ss += lane_xor_f(ss, o, lane);
    smax = fmaxf(smax, lane_xor_f(smax, o, lane));
  }
  if (lane == 0) {
    red[0][wave] = ss;
    red[1][wave] = smax;
  }
  __syncthreads();
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < KPT; ++i) acc = fmaf(m[i], q[wave * KPT + i], acc);
  part[wave][lane] = acc;
  __syncthreads();
  if (tid < 64) vals[tid] = (part[0][tid] + part[1][tid]) + (part[2][tid] + part[3][tid]);
  const float nq = sqrtf((red[0][0] + red[0][1]) + (red[0][2] + red[0][3]));
  const int npk = n_walsh(a.k.bq);
  double amax = 0.0;
  for (int p = 0; p < npk; ++p) amax = fmax(amax, fabs(a.walsh_k[p]));
  const double scale =
      sgn ? double(fmaxf(fmaxf(red[1][0], red[1][1]), fmaxf(red[1][2], red[1][3]))) : amax;
  const int E = fix_exp(scale * double(nq) * (1.0 + 0x1p-10));
  __syncthreads();
  // entry = (plane, chunk c, lane group g, digit l): 16 bytes for VGPR s, byte i.
  // Lane group g owns plane words g, g + 4, ...; chunk c takes word g + 4 (c >> 1)
  // and its nibble c & 1: byte i of VGPR s is coordinate 32 (g + 4 (c >> 1)) + 8 i + s + 4 (c & 1).
  // The slice holds words c0 / 32 and c0 / 32 + 1, both nibbles: 4 (g, c) pairs.
  uint4 *op = reinterpret_cast<uint4 *>(static_cast<unsigned char *>(a.qop) +
                                        (size_t(b * a.Hkv + kvh) * RB + rb) * 5 * C * kWave * 16);
  const int nplane = sgn ? 1 : npk;
  if (tid < nplane * 16) {
    const int l = tid & 3, hw = (tid >> 2) & 3, pidx = tid >> 4;
    const int w = c0 / 32 + (hw >> 1), h = hw & 1, g = w & 3, c = 2 * (w >> 2) + h;
    const float wk = sgn ? 1.0f : static_cast<float>(a.walsh_k[pidx]);
    uint32_t wv[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int sv = 0; sv < 4; ++sv)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = 32 * w + 8 * i + sv + 4 * h;
        const int32_t F = static_cast<int32_t>(rintf(ldexpf(wk * vals[j - c0], E - sv)));
        wv[sv] |= ((digits(F) >> (8 * l)) & 0xFFu) << (8 * i);
      }
    const int slot = sgn ? kSigPlane : pidx;
    op[(size_t(slot) * C + c) * kWave + 16 * g + row0 + l] = uint4{wv[0], wv[1], wv[2], wv[3]};
  }
  if (tid == 0 && (t == 0 || t == D / 64)) {
    // alpha (Walsh planes) or beta (sign plane, 0 without one): the scale of the digit sums
    const double base = a.qbase;  // sm_scale log2(e) (scores in base 2), or 1 for raw scores
    int32_t *qc = a.qconst + size_t(bh) * 8;
    if (sgn) qc[5] = __float_as_int(static_cast<float>(ldexp(base * double(a.kappa), -E)));
    else qc[4] = __float_as_int(static_cast<float>(ldexp(base, -E)));
    if (!sgn && !a.k.sketch) qc[5] = 0;
  }
}

// Query prep for many query heads: block (group of 8 heads, slice t), the same
// work as decode_qprep_fast for each head, with the slice of the transposed
// matrix read once for the group.
template <int D>
__global__ __launch_bounds__(256) void decode_qprep_grouped(DecodeArgs a, int nq) {
  constexpr int C = D / 64, NSL = 2 * D / 64, KPT = D / 4, HG = 8;
  __shared__ float q[HG][D];
  __shared__ float part[HG][4][64];
  __shared__ float vals[HG][64];
  __shared__ float qn[HG];
  __shared__ float red[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = blockIdx.x / NSL, t = blockIdx.x % NSL;
  const bool sgn = t >= D / 64;
  if (sgn && !a.k.sketch) return;  // no sign plane
  const int c0 = (sgn ? t - D / 64 : t) * 64;
  const float *mt = (sgn ? a.projT : a.rotT) + c0 + lane + size_t(wave) * KPT * D;
  float m[KPT];
#pragma unroll
  for (int i = 0; i < KPT; ++i) m[i] = mt[size_t(i) * D];
  float smax = 0.0f;
  if (sgn)
    for (int j = tid; j < D; j += 256) smax = fmaxf(smax, a.stnorm[j]);
  for (int i = tid; i < HG * D; i += 256) {
    const int h = i / D, j = i % D, bh = grp * HG + h;
    q[h][j] = bh < nq ? load_q(a.q, a.dtype, size_t(bh) * D + j) : 0.0f;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) smax = fmaxf(smax, lane_xor_f(smax, o, lane));
  if (lane == 0) red[wave] = smax;
  __syncthreads();
  // ||q|| of heads HG / 4 wave ..
#pragma unroll
  for (int u = 0; u < HG / 4; ++u) {
    const int h = HG / 4 * wave + u;
    float ss = 0.0f;
    for (int j = lane; j < D; j += 64) ss = fmaf(q[h][j], q[h][j], ss);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) ss += lane_xor_f(ss, o, lane);
    if (lane == 0) qn[h] = sqrtf(ss);
  }
#pragma unroll
  for (int h = 0; h < HG; ++h) {
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < KPT; ++i) acc = fmaf(m[i], q[h][wave * KPT + i], acc);
    part[h][wave][lane] = acc;
  }
  __syncthreads();
  for (int i = tid; i < HG * 64; i += 256) {
    const int h = i >> 6, c = i & 63;
    vals[h][c] = (part[h][0][c] + part[h][1][c]) + (part[h][2][c] + part[h][3][c]);
  }
  const int npk = n_walsh(a.k.bq);
  double amax = 0.0;
  for (int p = 0; p < npk; ++p) amax = fmax(amax, fabs(a.walsh_k[p]));
  const double scale = sgn ? double(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]))) : amax;
  __syncthreads();
  const int nplane = sgn ? 1 : npk;
  for (int e = tid; e < HG * nplane * 16; e += 256) {
    const int h = e / (nplane * 16), r = e % (nplane * 16), bh = grp * HG + h;
    if (bh >= nq) continue;
    const int E = fix_exp(scale * double(qn[h]) * (1.0 + 0x1p-10));
    const int b = bh / a.Hq, hq = bh % a.Hq;
    const int kvh = hq / a.G, hl = hq % a.G, rb = hl >> 2, row0 = (hl & 3) * 4, RB = a.G / 4;
    uint4 *op = reinterpret_cast<uint4 *>(static_cast<unsigned char *>(a.qop) +
                                          (size_t(b * a.Hkv + kvh) * RB + rb) * 5 * C * kWave * 16);
    const int l = r & 3, hw = (r >> 2) & 3, pidx = r >> 4;
    const int w = c0 / 32 + (hw >> 1), hh = hw & 1, g = w & 3, c = 2 * (w >> 2) + hh;
    const float wk = sgn ? 1.0f : static_cast<float>(a.walsh_k[pidx]);
    uint32_t wv[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int sv = 0; sv < 4; ++sv)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = 32 * w + 8 * i + sv + 4 * hh;
        const int32_t F = static_cast<int32_t>(rintf(ldexpf(wk * vals[h][j - c0], E - sv)));
        wv[sv] |= ((digits(F) >> (8 * l)) & 0xFFu) << (8 * i);
      }
    const int slot = sgn ? kSigPlane : pidx;
    op[(size_t(slot) * C + c) * kWave + 16 * g + row0 + l] = uint4{wv[0], wv[1], wv[2], wv[3]};
  }
  if ((t == 0 || t == D / 64) && tid < HG) {
    const int bh = grp * HG + tid;
    if (bh < nq) {
      const int E = fix_exp(scale * double(qn[tid]) * (1.0 + 0x1p-10));
      const double base = a.qbase;  // sm_scale log2(e) (scores in base 2), or 1 for raw scores
      int32_t *qc = a.qconst + size_t(bh) * 8;
      if (sgn) qc[5] = __float_as_int(static_cast<float>(ldexp(base * double(a.kappa), -E)));
      else qc[4] = __float_as_int(static_cast<float>(ldexp(base, -E)));
      if (!sgn && !a.k.sketch) qc[5] = 0;
    }
  }
}

// ------------------------------------------------------------ split pass ---
// One 256-thread block per (split, kv head, sequence); a split holds at most
// kMaxT * 256 slots.  BQK / BQV: index bits of keys / values (compile time: the
// plane loops unroll without branches); the sign planes always run, with zero
// operands when a tensor has no sketch.
//
// Lane roles: lane = 16 grp + col.  In a score MFMA col is the token of a
// 16-token block and grp the lane group of the contraction (coordinates); the
// result gives lane (col, grp) the four digit sums of query head 4 rb + grp
// for that token.  In a value MFMA col is the coordinate of a 16-coordinate
// block and grp the token group of the contraction.
//
// Data movement: every wave streams its own chunks through a private ring of
// LDS slots with buffer loads that write LDS directly (16 bytes per lane, no
// VGPRs), one chunk fewer than the slots ahead of the one it computes on.  A wave's
// stream is its key tiles (tiles wave, wave + 4, ...: planes, signs, key and
// value scales, each a contiguous run of the token-major cache), then one value
// chunk per round (its quarter of the coordinates of the round's 8 value blocks,
// one 1 KB load per plane).  Loads complete in order, so a chunk has landed once
// at most (chunks issued after it) x (fewest loads in a chunk) remain.
//
// Scores never leave registers: the lane that scores (head, token) in phase 1
// is the lane that turns it into a weight in phase 2.
constexpr int kMaxT = 4;   // key tiles per wave and split: split <= 1024 slots

typedef unsigned u4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

// Raw buffer descriptor (SGPRs): base, no stride, `bytes` records (reads past
// them return 0), 32-bit data format.
__device__ inline u4 make_rsrc(const void *base, int bytes) {
  const unsigned long long p = reinterpret_cast<unsigned long long>(base);
  u4 r;
  r.x = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(p));
  r.y = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(p >> 32) & 0xFFFFu);
  r.z = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(bytes));
  r.w = 0x00020000u;
  return r;
}

__device__ inline unsigned lds_addr(const void *p) {
  return __builtin_amdgcn_readfirstlane(static_cast<unsigned>(reinterpret_cast<uintptr_t>((const lds_void *)p)));
}

// 16 (or 4) bytes per lane from the buffer straight into LDS at dst + 16 lane
// (4 lane); dst is wave-uniform (M0).  Every offset goes in the VGPR offset,
// which the buffer range check covers (the SGPR offset is 0).  Written as asm so that the compiler does
// not track these loads: it would otherwise wait for all of them before LDS
// accesses it cannot tell apart from the ring.  The instructions have no
// register results; the LDS they write is read only after an explicit vmcnt
// wait (wait_vm), and no load is issued into a slot before this wave's reads
// of it are complete (lgkmcnt(0) first).
__device__ inline void dma16(u4 r, unsigned dst, int voff, int soff) {
  asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(r), "s"(soff), "{m0}"(dst) : "memory");
}
__device__ inline void dma4(u4 r, unsigned dst, int voff, int soff) {
  asm volatile("buffer_load_dword %0, %1, %2 offen lds" ::"v"(voff), "s"(r), "s"(soff), "{m0}"(dst) : "memory");
}

// Wait until at most N vector-memory loads of this wave are outstanding.  The
// memory clobber keeps the compiler from moving LDS reads of the landed chunk
// above the wait.
template <int N>
__device__ inline void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Block barrier for LDS exchanges only: this wave's LDS operations are complete
// first, but its loads in flight into the ring are not waited for.
__device__ inline void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ inline uint32_t lds32(const unsigned char *p) { return *reinterpret_cast<const uint32_t *>(p); }

// Score digit sums to 2 x - k exactly, then fp32: x = lo + 2^16 hi with
// lo = c0 + 2^8 c1, hi = c2 + 2^8 c3, and k = 2^17 KH + KL (0 <= KL < 2^17), so
// 2 x - k = 2^17 (hi - KH) + (2 lo - KL), both parts exact in int32.
__device__ inline float score_sum(v4i c, int32_t KH, int32_t KL) {
  const int32_t lo = c.x + (c.y << 8), hi = c.z + (c.w << 8);
  return fmaf(static_cast<float>(hi - KH), 131072.0f, static_cast<float>(2 * lo - KL));
}

template <int D, int RB, int BQK, int BQV, bool DEEP>
struct SplitShape {
  static constexpr int C = D / 64, W = D / 32, NB = D / 64, NW = D / 128, G = 4 * RB;
  static constexpr int PK = BQK == 3 ? 4 : BQK, PV = BQV == 3 ? 4 : BQV;
  static constexpr int KREC = BQK * W * 4, KSREC = W * 4;  // key bytes per slot: planes, signs
  static constexpr int VREC = BQV * D * 4, VSREC = D * 4;  // value bytes per 32-slot block
  // key chunk: planes [64][KREC], signs [64][KSREC], key scales [64], value scales [64]
  static constexpr int K_SG = 64 * KREC, K_KS = K_SG + 64 * KSREC, K_VS = K_KS + 256, K_BYTES = K_VS + 256;
  // value chunk: [plane (BQV, then signs)][block 8][D / 4 words]
  static constexpr int VPL = 8 * D, V_BYTES = (BQV + 1) * VPL;
  static constexpr int SLOT = K_BYTES > V_BYTES ? K_BYTES : V_BYTES;
  static constexpr int NI_K = (BQK + 1) * NW + 2, NI_V = (BQV + 1) * NW;  // loads per chunk
  static constexpr int NI_MIN = NI_K < NI_V ? NI_K : NI_V;
  // Ring slots per wave and value operand buffers (round parity).  DEEP (one
  // head block, few work-groups: latency-bound) keeps two chunks in flight per
  // wave; otherwise the smaller LDS footprint fits more work-groups per CU, which
  // hides more (three or four per CU).
  static constexpr int SLOTS = DEEP ? 3 : 2;
  static constexpr int AWP = DEEP ? 2 : 1;
};

// SCORES: key scoring (tq_score_keys) -- phase 1 only, over key head a.kv_fixed,
// writing each score instead of the split's attention partial.
template <int D, int RB, int BQK, int BQV, bool DEEP, bool SCORES = false>
__global__ __launch_bounds__(256) void decode_partial_fast(DecodeArgs a) {
  using P = SplitShape<D, RB, BQK, BQV, DEEP>;
  constexpr int C = P::C, W = P::W, NB = P::NB, NW = P::NW, G = P::G, PK = P::PK, PV = P::PV;
  constexpr int KREC = P::KREC, KSREC = P::KSREC, VREC = P::VREC, VSREC = P::VSREC, AWP = P::AWP;
  constexpr int kSlots = P::SLOTS;
  __shared__ __attribute__((aligned(16))) unsigned char ring[4][kSlots][P::SLOT];
  // value A operands of a round: [round parity][part][tile][kgroup][rb][row][byte]
  __shared__ __attribute__((aligned(16))) unsigned char aw[AWP][2][4][4][RB][16][16];
  // per wave: the digit words of its tile (one part at a time) in operand byte order
  __shared__ __attribute__((aligned(16))) uint32_t fst[4][RB][4][64];
  __shared__ float redf[4][G];
  __shared__ float redv[4][2];
  __shared__ float mh_s[G];
  __shared__ float lh_s[G];

  // wave index in an SGPR: offsets derived from it feed buffer-load SGPR offsets
  // and the LDS base of the direct loads, which must be provably uniform
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, col = lane & 15,
            grp = lane >> 4;
  // Scoring: every query group reads the same keys, so the groups of one split
  // run back to back on one XCD (work-groups go round-robin over the 8 XCDs) and
  // all but the first find the split's keys in that XCD's L2.
  const int bx = blockIdx.x, b = blockIdx.z;
  const int split = SCORES ? (bx >> 3) / a.Hkv * 8 + (bx & 7) : bx;
  const int h = SCORES ? (bx >> 3) % a.Hkv : blockIdx.y;
  int64_t start, len;
  clip_seq(a, b, &start, &len);
  const int S = a.split_tokens;
  const int64_t abase = (start & ~int64_t(63)) + int64_t(split) * S;
  const int64_t lo = abase > start ? abase : start;
  const int64_t hi = (abase + S) < (start + len) ? (abase + S) : (start + len);
  const int bh0 = b * a.Hq + h * G;
  const int stride = 2 + 2 * D;
  if (lo >= hi) {
    if (!SCORES && tid < G) {
      float *o = a.part + (size_t(bh0 + tid) * a.n_split + split) * stride;
      o[0] = -INFINITY;
      o[1] = 0.0f;
    }
    return;
  }
  const int ntile = static_cast<int>((hi - abase + 63) >> 6);
  const int vlo = static_cast<int>(lo - abase), vhi = static_cast<int>(hi - abase);  // valid slots
  const uint32_t sh = (grp & 1) ? 4u : 0u;  // value operand: odd nibbles, shift the word right by 4
  const int64_t kcap = a.k.cap, vcap = a.v.cap, vblocks = vcap >> 5;
  const bool skk = a.k.sketch != 0, skv = a.v.sketch != 0;
  const int kslots = static_cast<int>((kcap - abase) < S ? (kcap - abase) : S);
  const int64_t blk0 = abase >> 5;
  const int vblk = static_cast<int>((vblocks - blk0) < (S >> 5) ? (vblocks - blk0) : (S >> 5));
  const int hk = SCORES ? a.kv_fixed : h;  // key head
  const u4 rk = make_rsrc(a.k.idx + (int64_t(hk) * kcap + abase) * BQK * W, kslots * KREC);
  const u4 rks = make_rsrc(skk ? a.k.sgn + (int64_t(hk) * kcap + abase) * W : a.k.idx, skk ? kslots * KSREC : 0);
  const u4 rkc = make_rsrc(a.k.scl + (int64_t(hk) * kcap + abase) * 2, kslots * 4);
  const int vslots = static_cast<int>((vcap - abase) < S ? (vcap - abase) : S);
  // (scoring has no value cache: empty descriptors, whose loads return zeros)
  const u4 rvc = SCORES ? make_rsrc(a.k.scl, 0) : make_rsrc(a.v.scl + (int64_t(h) * vcap + abase) * 2, vslots * 4);
  const u4 rv = SCORES ? make_rsrc(a.k.idx, 0) : make_rsrc(a.v.idx + (int64_t(h) * vblocks + blk0) * BQV * D, vblk * VREC);
  const u4 rvs = SCORES || !skv ? make_rsrc(a.k.idx, 0) : make_rsrc(a.v.sgn + (int64_t(h) * vblocks + blk0) * D, vblk * VSREC);

  // ---- the wave's chunk stream ----
  const int nk = ntile > wave ? (ntile - wave + 3) >> 2 : 0;  // key tiles of this wave
  const int nr = SCORES ? 0 : (ntile + 3) >> 2;               // value rounds
  const int nch = nk + nr;
  // value chunk lane roles: lane -> (block, 16-byte piece) of the wave's coordinates
  const int vblkl = NW == 1 ? (lane >> 3) : (lane >> 4), vpiece = NW == 1 ? (lane & 7) : (lane & 15);
  auto issue = [&](int s) {
    const unsigned dst = lds_addr(&ring[wave][s % kSlots][0]);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (s < nk) {
      const int tile = wave + 4 * s;
#pragma unroll
      for (int i = 0; i < BQK * NW; ++i) dma16(rk, dst + 1024 * i, tile * 64 * KREC + 1024 * i + 16 * lane, 0);
#pragma unroll
      for (int i = 0; i < NW; ++i) dma16(rks, dst + P::K_SG + 1024 * i, tile * 64 * KSREC + 1024 * i + 16 * lane, 0);
      dma4(rkc, dst + P::K_KS, tile * 256 + 4 * lane, 0);
      dma4(rvc, dst + P::K_VS, tile * 256 + 4 * lane, 0);
    } else {
      const int r = s - nk;
#pragma unroll
      for (int p = 0; p <= BQV; ++p)
#pragma unroll
        for (int i = 0; i < NW; ++i) {
          const bool sg = p == BQV;
          const int rec = sg ? VSREC : VREC;
          const int voff = (8 * r + 4 * i + vblkl) * rec + (sg ? 0 : p * D * 4) + wave * D + 16 * vpiece;
          dma16(sg ? rvs : rv, dst + p * P::VPL + 1024 * i, voff, 0);
        }
    }
  };
  auto wait_chunk = [&](int s) {
    if (s + kSlots - 1 < nch) {
      if (SCORES) {
        // Scoring also stores 4 RB scores per lane and tile, unconditionally (one
        // store instruction each), between the chunk issues; vector loads and
        // stores complete in issue order, so the stores issued after chunk s --
        // those of the min(s, kSlots - 1) tiles since -- count behind it too.
        if (s == 0) wait_vm<(kSlots - 1) * P::NI_MIN>();
        else if (s == 1 || kSlots == 2) wait_vm<(kSlots - 1) * P::NI_MIN + 4 * RB>();
        else wait_vm<(kSlots - 1) * P::NI_MIN + 8 * RB>();
      } else {
        wait_vm<(kSlots - 1) * P::NI_MIN>();
      }
    } else {
      wait_vm<0>();
    }
  };

  // The first kSlots - 1 chunks, then the query operands and constants as plain
  // loads, which are waited for at once: the compiler does not see the direct
  // LDS loads, so any wait it placed later for a register load would count too
  // few loads behind it and drain the ring.  (Issues past the stream read past
  // the descriptors and land zeros in a free slot.)
#pragma unroll
  for (int s = 0; s < kSlots - 1; ++s) issue(s);
  v4i qa[RB][PK + 1][C];
  int2 qf[RB];  // per head: alpha and beta (fp32 bits)
  {
    const v4i *qop = static_cast<const v4i *>(a.qop) + size_t(b * a.Hkv + h) * RB * 5 * C * kWave;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
      for (int p = 0; p <= PK; ++p) {
        const int slot = p == PK ? kSigPlane : p;
#pragma unroll
        for (int c = 0; c < C; ++c)
          qa[rb][p][c] = (p < PK || skk) ? qop[((size_t(rb) * 5 + slot) * C + c) * kWave + lane] : v4i{0, 0, 0, 0};
      }
      qf[rb] = *reinterpret_cast<const int2 *>(a.qconst + size_t(bh0 + rb * 4 + grp) * 8 + 4);
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
      for (int p = 0; p <= PK; ++p)
#pragma unroll
        for (int c = 0; c < C; ++c)
          asm volatile("" ::"v"(qa[rb][p][c].x), "v"(qa[rb][p][c].y), "v"(qa[rb][p][c].z), "v"(qa[rb][p][c].w));
      asm volatile("" ::"v"(qf[rb].x), "v"(qf[rb].y));
    }
  }
  const uint32_t msk[4] = {0x01010101u, 0x02020202u, 0x04040404u, 0x08080808u};
  const v4i ones = {static_cast<int>(msk[0]), static_cast<int>(msk[1]), static_cast<int>(msk[2]),
                    static_cast<int>(msk[3])};
  // The +-1 corrections k = sum_j F_j 2^shift_j of the index planes (summed) and
  // of the sign plane: the query operands against all-ones bit planes, exact
  // digit sums, split as k = 2^17 KH + KL with 0 <= KL < 2^17.
  int32_t khi[RB], kli[RB], khs[RB], kls[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    v4i ci = {0, 0, 0, 0}, cs = {0, 0, 0, 0};
#pragma unroll
    for (int c = 0; c < C; ++c) {
#pragma unroll
      for (int p = 0; p < PK; ++p) ci = mfma(qa[rb][p][c], ones, ci);
      cs = mfma(qa[rb][PK][c], ones, cs);
    }
    const int64_t ki = int64_t(ci.x) + (int64_t(ci.y) << 8) + (int64_t(ci.z) << 16) + (int64_t(ci.w) << 24);
    const int64_t ks = int64_t(cs.x) + (int64_t(cs.y) << 8) + (int64_t(cs.z) << 16) + (int64_t(cs.w) << 24);
    khi[rb] = static_cast<int32_t>(ki >> 17);
    kli[rb] = static_cast<int32_t>(ki & 0x1FFFF);
    khs[rb] = static_cast<int32_t>(ks >> 17);
    kls[rb] = static_cast<int32_t>(ks & 0x1FFFF);
  }

  // ---- phase 1: scores of this wave's key tiles, kept in registers ----
  float sreg[kMaxT][4][RB];
  uint32_t vreg[kMaxT][4];  // value scales of the same tokens, for phase 2
  float mloc[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) mloc[rb] = -INFINITY;
  float vnumax = 0.0f, vrhomax = 0.0f;
#pragma unroll
  for (int kt = 0; kt < kMaxT; ++kt) {
    if (kt < nk) {
      issue(kt + kSlots - 1);
      wait_chunk(kt);
      const unsigned char *sl = &ring[wave][kt % kSlots][0];
      const int tile = wave + 4 * kt;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int tok = nb * 16 + col, t = tile * 64 + tok;
        const bool valid = t >= vlo && t < vhi;
        // lane group grp holds words grp, grp + 4, ... of the token's planes
        uint32_t wd[3][NW], ws[NW];
#pragma unroll
        for (int u = 0; u < NW; ++u) {
#pragma unroll
          for (int p = 0; p < 3; ++p) wd[p][u] = p < BQK ? lds32(sl + tok * KREC + p * W * 4 + (grp + 4 * u) * 4) : 0u;
          ws[u] = lds32(sl + P::K_SG + tok * KSREC + (grp + 4 * u) * 4);
        }
        const uint32_t ksc = lds32(sl + P::K_KS + 4 * tok), vsc = lds32(sl + P::K_VS + 4 * tok);
        v4i acc_i[RB], acc_s[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) acc_i[rb] = acc_s[rb] = v4i{0, 0, 0, 0};
#pragma unroll
        for (int c = 0; c < C; ++c) {
#pragma unroll
          for (int p = 0; p < PK; ++p) {
            const v4i B = expand(plane_word<4>(p, wd[0][c >> 1], wd[1][c >> 1], wd[2][c >> 1]), 4u * (c & 1), msk);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) acc_i[rb] = mfma(qa[rb][p][c], B, acc_i[rb]);
          }
          const v4i B = expand(ws[c >> 1], 4u * (c & 1), msk);
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) acc_s[rb] = mfma(qa[rb][PK][c], B, acc_s[rb]);
        }
        const float knu = f16v(ksc), krho = f16v(ksc >> 16);
        vreg[kt][nb] = vsc;
        vnumax = fmaxf(vnumax, valid ? f16v(vsc) : 0.0f);
        vrhomax = fmaxf(vrhomax, valid ? f16v(vsc >> 16) : 0.0f);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const float ri = score_sum(acc_i[rb], khi[rb], kli[rb]);
          const float rs = score_sum(acc_s[rb], khs[rb], kls[rb]);
          float sv = fmaf(knu * __int_as_float(qf[rb].x), ri, (krho * __int_as_float(qf[rb].y)) * rs);
          if (SCORES) {
            // stored at once (16 consecutive scores per row and lane group), by every
            // lane: a slot outside the range writes a per-lane dummy word instead, so
            // that the number of stores per tile is fixed for the ring's waits
            float *dst = valid ? a.scores + (size_t(bh0 + rb * 4 + grp) * a.score_ld + (abase + t - start))
                               : a.score_dummy + lane;
            *dst = sv;
            continue;
          }
          sv = valid ? sv : -INFINITY;
          sreg[kt][nb][rb] = sv;
          mloc[rb] = fmaxf(mloc[rb], sv);
        }
      }
    }
  }
  if (SCORES) {
    // every load this wave issued has landed before it ends (the ring is LDS)
    wait_vm<0>();
    return;
  }
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) mloc[rb] = fmaxf(mloc[rb], lane_xor_f(mloc[rb], o, lane));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    vnumax = fmaxf(vnumax, lane_xor_f(vnumax, o, lane));
    vrhomax = fmaxf(vrhomax, lane_xor_f(vrhomax, o, lane));
  }
  if (col == 0)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) redf[wave][rb * 4 + grp] = mloc[rb];
  if (lane == 0) {
    redv[wave][0] = vnumax;
    redv[wave][1] = vrhomax;
  }
  lds_barrier();
  if (tid < G) mh_s[tid] = fmaxf(fmaxf(redf[0][tid], redf[1][tid]), fmaxf(redf[2][tid], redf[3][tid]));
  const float vn_all = fmaxf(fmaxf(redv[0][0], redv[1][0]), fmaxf(redv[2][0], redv[3][0]));
  const float vr_all = fmaxf(fmaxf(redv[0][1], redv[1][1]), fmaxf(redv[2][1], redv[3][1]));
  const int Ew = fix_exp(vn_all), Ewp = fix_exp(vr_all);
  lds_barrier();
  float mh[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) mh[rb] = mh_s[rb * 4 + grp];

  // ---- phase 2: per round of 4 tiles, weights to digits, then value MFMAs ----
  // av[p] accumulates digit sums of weight x bit-plane p (slot PV: sign plane,
  // residual weights); ak[part] accumulates weight x 1 (the all-ones plane),
  // which the +-1 form of every plane needs.  Every wave runs every tile of a
  // round, so each wave's ak is complete.
  v4i av[PV + 1][NB][RB], ak[2][RB];
#pragma unroll
  for (int p = 0; p <= PV; ++p)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) av[p][nb][rb] = v4i{0, 0, 0, 0};
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) ak[0][rb] = ak[1][rb] = v4i{0, 0, 0, 0};
  float lloc[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) lloc[rb] = 0.0f;
#pragma unroll
  for (int r = 0; r < kMaxT; ++r) {
    if (r < nr) {
      const int s = nk + r, par = AWP == 2 ? (r & 1) : 0;
      if (s + kSlots - 1 < nch) issue(s + kSlots - 1);
      if (r < nk) {
        // weights of this wave's tile 4 r + wave (its key tile r): lane (col, grp)
        // takes token nb 16 + col of head rb 4 + grp; its digit words go to the
        // wave's staging block at the token's operand byte position 16 q + 4 sft + i
        // (lane group q of the value operand, word sft, byte i): the weight's
        // first, then the residual weight's
        const int tile = 4 * r + wave;
        uint32_t dres[4][RB];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const int w64 = nb * 16 + col, t = tile * 64 + w64;
          const bool valid = t >= vlo && t < vhi;
          const float vnu = valid ? f16v(vreg[r][nb]) : 0.0f, vrho = valid ? f16v(vreg[r][nb] >> 16) : 0.0f;
          const int sft = w64 & 3, bi = (w64 >> 3) & 3, q = 2 * (w64 >> 5) + ((w64 >> 2) & 1);
          const int pos = 16 * q + 4 * sft + bi;
          const float sw = ldexpf(vnu, Ew - sft), swp = ldexpf(vrho, Ewp - sft);
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            const float Pw = valid ? __builtin_amdgcn_exp2f(sreg[r][nb][rb] - mh[rb]) : 0.0f;
            lloc[rb] += Pw;
            // truncation toward zero: |error| < 1 unit of 2^-Ew, far below the
            // 24-bit resolution of the float weight itself
            fst[wave][rb][grp][pos] = digits(static_cast<int32_t>(Pw * sw));
            dres[nb][rb] = digits(static_cast<int32_t>(Pw * swp));
          }
        }
        // operand of lane (row col, group grp): row = (head, digit l); word sft
        // gathers digit l of the four staged words 16 grp + 4 sft + (0..3)
        const int hd = col >> 2, l = col & 3;
        const uint32_t sel = uint32_t(l) | (uint32_t(4 + l) << 8) | 0x0C0C0000u;
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          if (x == 1) {
            // the staged words of part 0 have been read (this wave's LDS operations
            // complete in order): stage the residual weights in their place
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
              const int w64 = nb * 16 + col;
              const int pos = 16 * (2 * (w64 >> 5) + ((w64 >> 2) & 1)) + 4 * (w64 & 3) + ((w64 >> 3) & 3);
#pragma unroll
              for (int rb = 0; rb < RB; ++rb) fst[wave][rb][grp][pos] = dres[nb][rb];
            }
          }
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            uint32_t wv[4];
#pragma unroll
            for (int sv = 0; sv < 4; ++sv) {
              const uint4 f = *reinterpret_cast<const uint4 *>(&fst[wave][rb][hd][16 * grp + 4 * sv]);
              const uint32_t lo2 = __builtin_amdgcn_perm(f.y, f.x, sel), hi2 = __builtin_amdgcn_perm(f.w, f.z, sel);
              wv[sv] = __builtin_amdgcn_perm(hi2, lo2, 0x05040100u);
            }
            *reinterpret_cast<uint4 *>(&aw[par][x][wave][grp][rb][col][0]) = uint4{wv[0], wv[1], wv[2], wv[3]};
          }
        }
      }
      lds_barrier();
      wait_chunk(s);
      const unsigned char *sl = &ring[wave][s % kSlots][0];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        if (4 * r + tt >= ntile) break;
        v4i aw0[RB], aw1[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          aw0[rb] = *reinterpret_cast<const v4i *>(&aw[par][0][tt][grp][rb][col][0]);
          aw1[rb] = *reinterpret_cast<const v4i *>(&aw[par][1][tt][grp][rb][col][0]);
          ak[0][rb] = mfma(aw0[rb], ones, ak[0][rb]);
          ak[1][rb] = mfma(aw1[rb], ones, ak[1][rb]);
        }
        // words of coordinates col NB .. col NB + NB - 1 (of the wave's quarter) in
        // value block 2 tt + grp / 2 of the round
        const unsigned char *vb = sl + (2 * tt + (grp >> 1)) * D + col * NB * 4;
        uint32_t vw[3][NB], vs[NB];
#pragma unroll
        for (int p = 0; p <= BQV; ++p) {
          uint32_t t4[NB];
          if constexpr (NB == 2) {
            const uint2 v2 = *reinterpret_cast<const uint2 *>(vb + p * P::VPL);
            t4[0] = v2.x;
            t4[1] = v2.y;
          } else {
            const uint4 v4 = *reinterpret_cast<const uint4 *>(vb + p * P::VPL);
            t4[0] = v4.x;
            t4[1] = v4.y;
            t4[2] = v4.z;
            t4[3] = v4.w;
          }
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            if (p == BQV) vs[nb] = t4[nb];
            else vw[p][nb] = t4[nb];
          }
        }
#pragma unroll
        for (int p = BQV; p < 3; ++p)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) vw[p][nb] = 0u;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
          for (int p = 0; p < PV; ++p) {
            const v4i B = expand(plane_word<4>(p, vw[0][nb], vw[1][nb], vw[2][nb]), sh, msk);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) av[p][nb][rb] = mfma(aw0[rb], B, av[p][nb][rb]);
          }
          const v4i B = expand(vs[nb], sh, msk);
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) av[PV][nb][rb] = mfma(aw1[rb], B, av[PV][nb][rb]);
        }
      }
      // with two operand buffers the next round writes the other one, and the
      // round after that is behind the next round's barrier; with one, wait here
      if (AWP == 1) lds_barrier();
    }
  }

  // ---- l over the block, then write this split's partial ----
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) lloc[rb] += lane_xor_f(lloc[rb], o, lane);
  if (col == 0)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) redf[wave][rb * 4 + grp] = lloc[rb];
  lds_barrier();
  if (tid < G) lh_s[tid] = (redf[0][tid] + redf[1][tid]) + (redf[2][tid] + redf[3][tid]);
  lds_barrier();
  const int j0 = wave * (D / 4) + col * NB;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int head = rb * 4 + grp;
    float *o = a.part + (size_t(bh0 + head) * a.n_split + split) * stride;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      double acc = 0.0;
#pragma unroll
      for (int p = 0; p < PV; ++p) acc += a.walsh_v[p] * pm_form(av[p][nb][rb], ak[0][rb]);
      o[2 + j0 + nb] = static_cast<float>(ldexp(acc, -Ew));
      o[2 + D + j0 + nb] = skv ? static_cast<float>(ldexp(pm_form(av[PV][nb][rb], ak[1][rb]), -Ewp)) : 0.0f;
    }
    if (wave == 0 && col == 0) {
      o[0] = mh[rb] * 0.69314718055994531f;  // natural-log units for the merge
      o[1] = lh_s[head];
    }
  }
}

// ----------------------------------------------------------------- merge ---
// out = (Pi^T A + kappa S^T B) / l, where (A, B) and l merge the split partials
// by log-sum-exp.  Block (head, cs) computes the CPB x 64 outputs from 64 CPB cs
// on (CPB = d / 64, one block per head, when there are heads enough to fill the
// chip; else CPB = 1):
//  1. the split maxima and sums: M = max m_s over splits with tokens, weights
//     w_s = exp(m_s - M) (0 for a split with no tokens, whose (A, B) are
//     unwritten), l = sum w_s l_s; the weights go to LDS.
//  2. thread (sg, e) sums w_s x_s for element e of (A, B) over splits sg,
//     sg + SGN, ...; its loads are issued before step 1 (they do not depend on
//     the weights), as are the matrix loads of step 3.  The split groups are
//     added in LDS.
//  3. per group of 64 columns, thread (kq, jj) takes rows kq, kq + 8, ... of
//     [Pi ; S] (2 d rows) at the group's column jj; the 8 row groups are added
//     in LDS.
// Every block of a head recomputes steps 1-2 so that no block waits on another.
constexpr int kMaxSplits = 2048;

template <int D, int CPB>
__global__ __launch_bounds__(512) void decode_merge_fast(DecodeArgs a) {
  constexpr int NT = 512, SGN = NT / (2 * D), CHS = 32;  // split groups, split loads per chunk
  constexpr int RPT = 2 * D / 8;                         // matrix rows per thread
  __shared__ float ws_l[kMaxSplits], ls_l[kMaxSplits];
  __shared__ float red[8];
  __shared__ float accg[SGN][2 * D];
  __shared__ float prj[8][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int ncs = D / (64 * CPB);
  const int bh = blockIdx.x / ncs, cs = blockIdx.x % ncs;
  const int stride = 2 + 2 * D, ns = a.n_split;
  const float *base = a.part + size_t(bh) * ns * stride;
  // step 3's matrix column: rows kq + 8 i of [Pi ; S]
  const int jj = tid & 63, kq = tid >> 6;
  float mrow[RPT];
  auto load_rows = [&](int col) {
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int k = kq + 8 * i;
      mrow[i] = k < D ? a.rot[size_t(k) * D + col] : a.proj[size_t(k - D) * D + col];
    }
  };
  load_rows(64 * CPB * cs + jj);
  // step 2's first chunk of elements
  const int e = tid % (2 * D), sg = tid / (2 * D);
  float x[CHS];
#pragma unroll
  for (int u = 0; u < CHS; ++u) {
    const int s = sg + SGN * u;
    x[u] = s < ns ? base[size_t(s) * stride + 2 + e] : 0.0f;
  }
  // step 1
  float mmax = -INFINITY;
  for (int s = tid; s < ns; s += NT) {
    const float ms = base[size_t(s) * stride], ls = base[size_t(s) * stride + 1];
    ws_l[s] = ls > 0.0f ? ms : -INFINITY;
    ls_l[s] = ls > 0.0f ? ls : 0.0f;
    mmax = fmaxf(mmax, ws_l[s]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mmax = fmaxf(mmax, lane_xor_f(mmax, o, lane));
  if (lane == 0) red[wave] = mmax;
  __syncthreads();
  float M = red[0];
#pragma unroll
  for (int w = 1; w < 8; ++w) M = fmaxf(M, red[w]);
  __syncthreads();
  float lsum = 0.0f;
  for (int s = tid; s < ns; s += NT) {
    const float ms = ws_l[s];
    const float w = ms > -INFINITY ? expf(ms - M) : 0.0f;
    lsum = fmaf(w, ls_l[s], lsum);
    ws_l[s] = w;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) lsum += lane_xor_f(lsum, o, lane);
  if (lane == 0) red[wave] = lsum;
  __syncthreads();
  float l = 0.0f;
#pragma unroll
  for (int w = 0; w < 8; ++w) l += red[w];
  // step 2
  float acc = 0.0f;
  for (int s0 = 0; s0 < ns; s0 += SGN * CHS) {
    if (s0 > 0)
#pragma unroll
      for (int u = 0; u < CHS; ++u) {
        const int s = s0 + sg + SGN * u;
        x[u] = s < ns ? base[size_t(s) * stride + 2 + e] : 0.0f;
      }
#pragma unroll
    for (int u = 0; u < CHS; ++u) {
      const int s = s0 + sg + SGN * u;
      const float w = s < ns ? ws_l[s] : 0.0f;
      acc = w > 0.0f ? fmaf(w, x[u], acc) : acc;  // a split without tokens has stale (A, B)
    }
  }
  accg[sg][e] = e < D ? acc : a.kappa * acc;
  __syncthreads();
  // step 3
  float v[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    v[i] = 0.0f;
#pragma unroll
    for (int g = 0; g < SGN; ++g) v[i] += accg[g][kq + 8 * i];
  }
#pragma unroll 1
  for (int cg = 0; cg < CPB; ++cg) {
    const int col0 = 64 * (CPB * cs + cg);
    if (cg > 0) {
      load_rows(col0 + jj);
      __syncthreads();  // prj of the previous group has been read
    }
    float pj = 0.0f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) pj = fmaf(mrow[i], v[i], pj);
    prj[kq][jj] = pj;
    __syncthreads();
    if (tid < 64) {
      float o = 0.0f;
#pragma unroll
      for (int g = 0; g < 8; ++g) o += prj[g][tid];
      a.out[size_t(bh) * D + col0 + tid] = l > 0.0f ? o / l : 0.0f;
    }
  }
}

// Merge for many query heads: block = group of 8 heads, all d outputs.  The
// per-head blocks above read the whole projection matrix once per head; here
// one wave merges one head's splits (lane e holds elements e EPT .. e EPT + EPT - 1
// of (A, B), a running maximum over chunks of CHS splits whose loads are issued
// together), and the block then applies [Pi ; S], 64 columns at a time, to all
// eight heads, reading it once per group.
template <int D>
__global__ __launch_bounds__(512) void decode_merge_grouped(DecodeArgs a, int nq) {
  constexpr int HG = 8, EPT = 2 * D / 64, CHS = D == 128 ? 24 : 4, RPT = 2 * D / 8;
  __shared__ __attribute__((aligned(16))) float ab[HG][2 * D];
  __shared__ float lg[HG];
  __shared__ float prj[HG][8][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = blockIdx.x;
  const int stride = 2 + 2 * D, ns = a.n_split;
  // the projection's first matrix column group, rows kq + 8 i of [Pi ; S], issued first
  const int jj = lane, kq = wave;
  float mrow[RPT];
  auto load_rows = [&](int col) {
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int k = kq + 8 * i;
      mrow[i] = k < D ? a.rot[size_t(k) * D + col] : a.proj[size_t(k - D) * D + col];
    }
  };
  load_rows(jj);
  // one head per wave
  const int bh = grp * HG + wave;
  if (bh < nq) {
    const float *base = a.part + size_t(bh) * ns * stride;
    float m_run = -INFINITY, l_run = 0.0f, acc[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) acc[e] = 0.0f;
    for (int s0 = 0; s0 < ns; s0 += CHS) {
      float pm[CHS], pl[CHS], x[CHS][EPT];
#pragma unroll
      for (int u = 0; u < CHS; ++u) {
        const int s = s0 + u;
        pm[u] = -INFINITY;
        pl[u] = 0.0f;
#pragma unroll
        for (int e = 0; e < EPT; ++e) x[u][e] = 0.0f;
        if (s < ns) {
          const float *p = base + size_t(s) * stride;
          pm[u] = p[0];
          pl[u] = p[1];
          // element 2 + e sits 8 bytes past a 16-byte boundary: float2 pairs
#pragma unroll
          for (int e = 0; e < EPT; e += 2) {
            const float2 v2 = *reinterpret_cast<const float2 *>(p + 2 + lane * EPT + e);
            x[u][e] = v2.x;
            x[u][e + 1] = v2.y;
          }
        }
      }
      float mc = m_run;
#pragma unroll
      for (int u = 0; u < CHS; ++u) mc = pl[u] > 0.0f ? fmaxf(mc, pm[u]) : mc;
      if (mc > -INFINITY) {
        const float co = m_run > -INFINITY ? expf(m_run - mc) : 0.0f;
        l_run *= co;
#pragma unroll
        for (int e = 0; e < EPT; ++e) acc[e] *= co;
#pragma unroll
        for (int u = 0; u < CHS; ++u) {
          // a split without tokens has stale (A, B)
          const float w = pl[u] > 0.0f ? expf(pm[u] - mc) : 0.0f;
          l_run = fmaf(w, pl[u], l_run);
#pragma unroll
          for (int e = 0; e < EPT; ++e) acc[e] = w > 0.0f ? fmaf(w, x[u][e], acc[e]) : acc[e];
        }
        m_run = mc;
      }
    }
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const int el = lane * EPT + e;
      ab[wave][el] = el < D ? acc[e] : a.kappa * acc[e];
    }
    if (lane == 0) lg[wave] = l_run;
  }
  __syncthreads();
#pragma unroll 1
  for (int cs = 0; cs < D / 64; ++cs) {
    if (cs > 0) {
      load_rows(64 * cs + jj);
      __syncthreads();  // prj of the previous column group has been read
    }
#pragma unroll 1
    for (int h = 0; h < HG; ++h) {
      float pj = 0.0f;
#pragma unroll
      for (int i = 0; i < RPT; ++i) pj = fmaf(mrow[i], ab[h][kq + 8 * i], pj);
      prj[h][kq][jj] = pj;
    }
    __syncthreads();
    const int h = wave, j = lane, bho = grp * HG + h;
    if (bho < nq) {
      float o = 0.0f;
#pragma unroll
      for (int g = 0; g < 8; ++g) o += prj[h][g][j];
      const float l = lg[h];
      a.out[size_t(bho) * D + 64 * cs + j] = l > 0.0f ? o / l : 0.0f;
    }
  }
}

template <int D, int RB, int BQK, bool DEEP>
int launch_partial_bv(int bqv, const DecodeArgs &a, hipStream_t s) {
  const dim3 grid(a.n_split, a.Hkv, a.batch);
  if (a.split_tokens > kMaxT * 256 || a.n_split > kMaxSplits) return 1;
  switch (bqv) {
    case 1: hipLaunchKernelGGL((decode_partial_fast<D, RB, BQK, 1, DEEP>), grid, dim3(256), 0, s, a); return 0;
    case 2: hipLaunchKernelGGL((decode_partial_fast<D, RB, BQK, 2, DEEP>), grid, dim3(256), 0, s, a); return 0;
    case 3: hipLaunchKernelGGL((decode_partial_fast<D, RB, BQK, 3, DEEP>), grid, dim3(256), 0, s, a); return 0;
    default: return 1;
  }
}

template <int D, int RB, bool DEEP>
int launch_partial(const DecodeArgs &a, hipStream_t s) {
  switch (a.k.bq) {
    case 1: return launch_partial_bv<D, RB, 1, DEEP>(a.v.bq, a, s);
    case 2: return launch_partial_bv<D, RB, 2, DEEP>(a.v.bq, a, s);
    case 3: return launch_partial_bv<D, RB, 3, DEEP>(a.v.bq, a, s);
    default: return 1;
  }
}

template <int D>
int launch_fast_d(int rb, const DecodeArgs &a, hipStream_t s) {
  const unsigned nq = static_cast<unsigned>(a.batch * a.Hq);
  if (nq >= 512)
    hipLaunchKernelGGL(decode_qprep_grouped<D>, dim3((nq + 7) / 8 * (2 * D / 64)), dim3(256), 0, s, a, int(nq));
  else hipLaunchKernelGGL(decode_qprep_fast<D>, dim3(nq * (2 * D / 64)), dim3(256), 0, s, a);
  // one head block and at most about two work-groups per CU: the deep ring
  const bool deep = int64_t(a.n_split) * a.Hkv * a.batch <= 1024;
  int e = rb == 2 ? launch_partial<D, 2, false>(a, s) : deep ? launch_partial<D, 1, true>(a, s)
                                                              : launch_partial<D, 1, false>(a, s);
  if (e) return e;
  // few splits per head: the projection matrix is the larger read, so heads share it
  if (nq >= 512 && a.n_split <= 64)
    hipLaunchKernelGGL(decode_merge_grouped<D>, dim3((nq + 7) / 8), dim3(512), 0, s, a, int(nq));
  else if (nq >= 128) hipLaunchKernelGGL((decode_merge_fast<D, D / 64>), dim3(nq), dim3(512), 0, s, a);
  else hipLaunchKernelGGL((decode_merge_fast<D, 1>), dim3(nq * (D / 64)), dim3(512), 0, s, a);
  return 0;
}

template <int D, int RB, int BQK, bool DEEP>
int launch_score_bq(const DecodeArgs &a, hipStream_t s) {
  // splits rounded up to a multiple of 8 (the XCD count); the extra work-groups
  // find an empty range and return
  const dim3 grid((a.n_split + 7) / 8 * 8 * a.Hkv, 1, a.batch);
  if (a.split_tokens > kMaxT * 256) return 1;
  hipLaunchKernelGGL((decode_partial_fast<D, RB, BQK, BQK, DEEP, true>), grid, dim3(256), 0, s, a);
  return 0;
}

template <int D>
int launch_score_d(const DecodeArgs &a, hipStream_t s) {
  const unsigned nq = static_cast<unsigned>(a.batch * a.Hq);
  if (nq >= 512)
    hipLaunchKernelGGL(decode_qprep_grouped<D>, dim3((nq + 7) / 8 * (2 * D / 64)), dim3(256), 0, s, a, int(nq));
  else hipLaunchKernelGGL(decode_qprep_fast<D>, dim3(nq * (2 * D / 64)), dim3(256), 0, s, a);
  const bool deep = int64_t(a.n_split) * a.Hkv * a.batch <= 1024;
  // groups of 16 queries (four row blocks) at d = 128, where their operands fit
  // in registers: each expansion of a key plane then feeds four MFMAs
  if constexpr (D == 128) {
    if (a.G == 16) switch (a.k.bq) {
      case 1: return deep ? launch_score_bq<D, 4, 1, true>(a, s) : launch_score_bq<D, 4, 1, false>(a, s);
      case 2: return deep ? launch_score_bq<D, 4, 2, true>(a, s) : launch_score_bq<D, 4, 2, false>(a, s);
      case 3: return deep ? launch_score_bq<D, 4, 3, true>(a, s) : launch_score_bq<D, 4, 3, false>(a, s);
      default: return 1;
    }
  }
  if (a.G != 8) return 1;
  switch (a.k.bq) {
    case 1: return deep ? launch_score_bq<D, 2, 1, true>(a, s) : launch_score_bq<D, 2, 1, false>(a, s);
    case 2: return deep ? launch_score_bq<D, 2, 2, true>(a, s) : launch_score_bq<D, 2, 2, false>(a, s);
    case 3: return deep ? launch_score_bq<D, 2, 3, true>(a, s) : launch_score_bq<D, 2, 3, false>(a, s);
    default: return 1;
  }
}

}  // namespace

int launch_score_fast(int d, const DecodeArgs &a, hipStream_t s) {
  int e = d == 128 ? launch_score_d<128>(a, s) : d == 256 ? launch_score_d<256>(a, s) : 1;
  if (e) return e;
  return hipGetLastError() != hipSuccess;
}

int launch_decode_fast(int d, int rb, const DecodeArgs &a, hipStream_t s) {
  int e = 1;
  if (d == 128) e = launch_fast_d<128>(rb, a, s);
  else if (d == 256) e = launch_fast_d<256>(rb, a, s);
  if (e) return e;
  return hipGetLastError() != hipSuccess;
}

}  // namespace tq
