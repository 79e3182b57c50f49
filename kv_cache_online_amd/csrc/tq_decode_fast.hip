// Decode attention over the packed caches on the CDNA4 matrix cores.
//
// The speed of decode over a compressed cache comes from moving fewer bytes
// (ast-softpro.ru, "Технология TurboQuant и её применение с локальными LLM",
// section 1.3).  On MI355X the vector ALU cannot keep up with HBM if every
// query head takes its own dot products with every unpacked coordinate, so the
// contractions of all G query heads of a kv head run on the matrix cores, with
// the packed bits as operands:
//
//  * Bit-plane operands.  A codebook value is an odd function of the +-1
//    bit-planes of its index (Walsh expansion: b' = 1, 2 are linear, b' = 3 adds
//    the triple product s0 s1 s2 = 2 (b0 ^ b1 ^ b2) - 1).  With s = 2 b - 1 a
//    dot product with a plane is 2 <v, b> - sum(v), so the products only need
//    0/1 bits.
//  * Scores: v_mfma_scale_f32_16x16x128_f8f6f4.  A key plane word masked four
//    ways is an fp4 (e2m1) operand of 32 coordinates (a set bit reads 0.5, 1 or
//    2); the queries are fp6 (e2m3) base-16 digits of 24-bit block fixed-point
//    numbers whose digit weights ride on the E8M0 block scales, so every digit
//    of every head sums into one fp32 accumulator row per (head, slot).
//  * Values: v_mfma_i32_16x16x64_i8, exact.  Packed value bits (a word shifted
//    right by 0 or 4, ANDed with 0x01010101 << k) are int8 operand bytes
//    bit << k, k = 0..3; the softmax weights times the value scales are
//    fixed-point integers F with |F| < 2^30, written as four signed base-256
//    digits (bytes of (F + 0x808080) ^ 0x808080), rows (query head, digit), and
//    recombined in float64 at the end of the split.
//  * Exact split maximum.  A split is at most 1280 slots; its scores stay in
//    the registers of the lanes that computed them, and the value pass runs
//    after the split's maximum is known, so the integer accumulators never need
//    rescaling.
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
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned short us2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kSigPlane = 4;     // operand / accumulator slot of the sign plane

// Floats per split partial record: m, l, two pad words, A [D], B [D] ((A, B) start
// 16-byte aligned, for 16-byte loads in the merge).
template <int D>
constexpr int part_stride() { return 4 + 2 * D; }

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

// fp4 (e2m1) B operand of a key plane word: dword r holds bits 4 i + r at nibble i,
// a set bit being 1, 1, 2, 2 for r = 0..3 (nibbles 0010, 0010, 0100, 0100).
__device__ inline v8i fp4_planes(uint32_t w) {
  return v8i{static_cast<int>((w << 1) & 0x22222222u), static_cast<int>(w & 0x22222222u),
             static_cast<int>(w & 0x44444444u), static_cast<int>((w >> 1) & 0x44444444u), 0, 0, 0, 0};
}

// One score product: A = six words of fp6 (e2m3) query digits, B = fp4 key bits,
// fp32 accumulate; the A block scale is byte q & 3 of sc[q >> 2] (E8M0), the B
// scale 1.  q is a constant once the caller's loops unroll, so the switch folds.
template <int N>
__device__ __forceinline__ v4f qmfma(const uint32_t (&A)[6], v8i B, v4f c, const uint32_t (&sc)[N], int q) {
  const v8i a = {static_cast<int>(A[0]), static_cast<int>(A[1]), static_cast<int>(A[2]),
                 static_cast<int>(A[3]), static_cast<int>(A[4]), static_cast<int>(A[5]), 0, 0};
  const int s = static_cast<int>(sc[q >> 2]);
  constexpr int kOne = 0x7F7F7F7F;  // E8M0 1.0 in every byte
  switch (q & 3) {
    case 0: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, B, c, 2, 4, 0, s, 0, kOne);
    case 1: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, B, c, 2, 4, 1, s, 0, kOne);
    case 2: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, B, c, 2, 4, 2, s, 0, kOne);
    default: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, B, c, 2, 4, 3, s, 0, kOne);
  }
}

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

// A wave-uniform read of memory that no kernel of the launch writes, through the
// scalar cache (constant address space): the clipping below then runs on the
// scalar unit instead of the vector ALU.
template <typename T>
__device__ inline T load_uniform(const T *p) {
  return *reinterpret_cast<const __attribute__((address_space(4))) T *>(reinterpret_cast<uintptr_t>(p));
}

__device__ inline void clip_seq(const DecodeArgs &a, int b, int64_t *start, int64_t *len) {
  const bool fixed = a.seq_start == nullptr;  // key scoring: one slot range, keys only
  int64_t s = fixed ? a.fix_start : load_uniform(a.seq_start + b);
  int64_t n = fixed ? a.fix_len : load_uniform(a.seq_len + b);
  const int64_t cap = fixed ? a.k.cap : a.k.cap < a.v.cap ? a.k.cap : a.v.cap;
  bool bad = false;
  if (n < 0) { n = 0; bad = true; }
  if (s < 0 || s > cap) { s = 0; n = 0; bad = true; }
  if (s + n > cap) { n = cap - s; bad = true; }
  if (!fixed && n > a.max_len) { n = a.max_len; bad = true; }  // the launch covers max_len slots
  if (bad && a.status && threadIdx.x == 0 && blockIdx.x == 0 && blockIdx.y == 0) atomicOr(a.status, TQ_FLAG_OUT_OF_RANGE);
  *start = s;
  *len = n;
}

// ------------------------------------------------------------- query prep ---
// Operands of the score products.  A key plane's bits meet the query in
// v_mfma_scale_f32_16x16x128_f8f6f4 with the bits as fp4 (e2m1) B operand and the
// query as fp6 (e2m3) A operand:
//
//  * B: lane (token col, lane group g) of chunk c takes plane word 4 c + g (its
//    32 coordinates) and masks it four ways: dword r holds bits 4 i + r at nibble
//    i ((w << 1) & 0x22222222, w & 0x22222222, w & 0x44444444,
//    (w >> 1) & 0x44444444), so a set bit is the fp4 value f_r = 1, 1, 2, 2.
//    Entry e = 8 r + i of the lane's 32 (its K index 32 g + e) is coordinate
//    32 (4 c + g) + 4 i + r.
//  * A: lane (row m, g) holds the same 32 coordinates.  Row m is (query head hl,
//    digit slot s), m = 4 (hl % 4) + S (hl / 4) + s with S = 16 / G slots, so the
//    accumulator lane that holds rows 4 g' .. 4 g' + 3 holds heads g' + 4 rb.
//    Entry e of a block of 32 carries the target T = 2 w v_j / f_r (v the
//    rotated or sketched query, w the Walsh coefficient times the score scale,
//    or kappa times it for the sign plane), as a 24-bit fixed-point number
//    F = rint(T 2^E), |F| < 2^24, with E from the block's largest |T|: F's
//    base-16 digits in
//    sign-magnitude form are e2m3 codes (code = sign << 5 | nibble, value
//    nibble / 8, exact), and digit l (of product l / S, slot l % S) carries the
//    E8M0 block scale 2^(4 l + 3 - E).
//
// The products then sum 2 w v_j b_j over a plane's coordinates in fp32, the
// rows of a head's slots adding up to its score; the split pass starts each
// accumulator at minus half the operand's product with all-ones planes (the +-1
// form 2 b - 1 of a bit) so that the sum is w <v, 2 b - 1>.  Each entry T is
// within 2^-24 of its block's largest |T| <= 2 |w| max|v|, so each term w v_j
// is within 2^-23 |w| max|v| and a plane's sum within 2^-16 |w| max|v| (d = 128;
// in practice the roundings are independent and far smaller); the fp32
// accumulation adds a few roundings of the partial sums.

// Pass 1, thread (plane p, word wsl of the slice, entry e) of one head: its
// target T (entry e of lane group "word" is coordinate 32 w + 4 (e & 7) + (e >> 3),
// whose key bit reads f = 1 for e >> 3 < 2, else 2), the block exponent from the
// word's largest |T| (the 32 threads of a word are one half of a wave), the
// fixed-point value F = rint(T 2^E), |F| < 2^24, and its six e2m3 digit codes
// (sign << 5 | nibble l) as bytes 0..5 of code[p][wsl][e]; E into Ex[p][wsl].
__device__ inline void query_fixed_point(const DecodeArgs &a, const float *vals, bool sgn, int idx,
                                         uint2 (*code)[2][32], int (*Ex)[2], int lane) {
  const int pidx = idx >> 6, wsl = (idx >> 5) & 1, e = idx & 31;
  const double wk = sgn ? (a.k.sketch ? a.qbase * double(a.kappa) : 0.0) : a.qbase * a.walsh_k[pidx];
  const float c = static_cast<float>((e >> 3) < 2 ? 2.0 * wk : wk);
  const float t = c * vals[32 * wsl + 4 * (e & 7) + (e >> 3)];
  float tmax = fabsf(t);
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) tmax = fmaxf(tmax, lane_xor_f(tmax, o, lane));
  const int E = tmax > 0.0f ? 23 - ilogbf(tmax) : 0;  // |T| 2^E < 2^24
  const float Fv = rintf(ldexpf(t, E));                // an integer, exact in fp32
  uint32_t mag = static_cast<uint32_t>(fabsf(Fv));
  mag = mag > 0xFFFFFFu ? 0xFFFFFFu : mag;             // rint may reach 2^24
  const uint32_t sg = Fv < 0.0f ? 0x20202020u : 0u;
  // nibbles 0..3 and 4..5 of mag, one per byte
  const uint32_t lo = (mag & 0xFu) | ((mag & 0xF0u) << 4) | ((mag & 0xF00u) << 8) | ((mag & 0xF000u) << 12);
  const uint32_t hi = ((mag >> 16) & 0xFu) | ((mag >> 12) & 0xF00u);
  code[pidx][wsl][e] = uint2{lo | sg, hi | (sg & 0x2020u)};
  if (e == 0) Ex[pidx][wsl] = E;
}

// Pass 2: one lane's operand for (plane pidx or the sign plane, word wsl of the
// slice, product i, slot s) of query head hl of group grp_idx (item enumerates
// them): digit l = S i + s of the 32 entries in 6-bit fields, and its block
// scale byte.
template <int D, int G>
__device__ void pack_query_operand(const DecodeArgs &a, const uint2 (*code)[2][32], const int (*Ex)[2], int c0,
                                   bool sgn, int npk, int grp_idx, int hl, int item) {
  constexpr int NW = D / 128, S = 16 / G, NM = (kQDigits + S - 1) / S;
  const int s = item % S, i = (item / S) % NM, wsl = (item / (S * NM)) & 1, pidx = item / (S * NM * 2);
  const int w = c0 / 32 + wsl, g = w & 3, c = w >> 2;
  const int m = 4 * (hl & 3) + S * (hl >> 2) + s, lane = 16 * g + m, l = S * i + s;
  uint32_t dw[6] = {0u, 0u, 0u, 0u, 0u, 0u};
  if (l < kQDigits) {
    const uint32_t *cw = reinterpret_cast<const uint32_t *>(code[pidx][wsl]) + (l >> 2);
    const uint32_t bs = 8 * (l & 3);
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const uint32_t cd = (cw[2 * e] >> bs) & 63u;
      const int pos = 6 * e, k = pos >> 5, sh = pos & 31;
      dw[k] |= cd << sh;
      if (sh > 26) dw[k + 1] |= cd >> (32 - sh);
    }
  }
  const int slot = sgn ? kSigPlane : pidx;
  uint32_t *op = a.qop + ((((size_t(grp_idx) * 5 + slot) * NW + c) * NM + i) * kWave + lane) * 8;
  *reinterpret_cast<uint4 *>(op) = uint4{dw[0], dw[1], dw[2], dw[3]};
  *reinterpret_cast<uint2 *>(op + 4) = uint2{dw[4], dw[5]};
  int sc = 127 + 4 * l + 3 - Ex[pidx][wsl];
  sc = sc < 0 ? 0 : sc > 254 ? 254 : sc;
  const int pslot = sgn ? npk : pidx;
  a.qscale[(size_t(grp_idx) * kWave + lane) * 32 + (pslot * NW + c) * NM + i] = static_cast<uint8_t>(sc);
}

template <int G>
__device__ inline int q_items(const DecodeArgs &a, bool sgn) {
  constexpr int S = 16 / G;
  return (sgn ? 1 : n_walsh(a.k.bq)) * 2 * ((kQDigits + S - 1) / S) * S;
}

// Block (sequence, query head, slice t) of 2 d / 64: slice t < d / 64 covers
// coordinates 64 t .. 64 t + 63 of q_rot = Pi q (the Walsh planes' operands),
// slice t >= d / 64 the same coordinates of q_s = S q (the sign plane's).  It
// computes its 64 products in fp32 (about 2^-24 relative error, far inside what
// the scores need) from the transposed matrices, so that a wave's loads are
// contiguous, and writes this head's rows of its operand entries.
template <int D, int G>
__global__ __launch_bounds__(256) void decode_qprep_fast(DecodeArgs a) {
  constexpr int NSL = 2 * D / 64, KPT = D / 4;
  __shared__ float q[D];
  __shared__ float part[4][64];
  __shared__ float vals[64];
  __shared__ uint2 fx[4][2][32];
  __shared__ int ex[4][2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bh = blockIdx.x / NSL, t = blockIdx.x % NSL;
  const int b = bh / a.Hq, hq = bh % a.Hq;
  const int kvh = hq / G, hl = hq % G;
  const bool sgn = t >= D / 64;
  const int c0 = (sgn ? t - D / 64 : t) * 64;
  // column c0 + lane of Pi^T or S^T, rows wave KPT .. wave KPT + KPT - 1
  const float *mt = (sgn ? a.projT : a.rotT) + c0 + lane + size_t(wave) * KPT * D;
  float m[KPT];
#pragma unroll
  for (int i = 0; i < KPT; ++i) m[i] = mt[size_t(i) * D];
  for (int j = tid; j < D; j += 256) q[j] = load_q(a.q, a.dtype, size_t(bh) * D + j);
  __syncthreads();
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < KPT; ++i) acc = fmaf(m[i], q[wave * KPT + i], acc);
  part[wave][lane] = acc;
  __syncthreads();
  if (tid < 64) vals[tid] = (part[0][tid] + part[1][tid]) + (part[2][tid] + part[3][tid]);
  __syncthreads();
  const int npk = n_walsh(a.k.bq), nplane = sgn ? 1 : npk;
  if (tid < nplane * 64) query_fixed_point(a, vals, sgn, tid, fx, ex, lane);
  __syncthreads();
  if (tid < q_items<G>(a, sgn)) pack_query_operand<D, G>(a, fx, ex, c0, sgn, npk, b * a.Hkv + kvh, hl, tid);
}

constexpr int kQPrepGroup = 4;  // query heads per block of the grouped query prep

// Query prep for many query heads: block (group of kQPrepGroup heads, slice t), the same
// work as decode_qprep_fast for each head, with the slice of the transposed
// matrix read once for the group.
template <int D, int G>
__global__ __launch_bounds__(256) void decode_qprep_grouped(DecodeArgs a, int nq) {
  constexpr int NSL = 2 * D / 64, KPT = D / 4, HG = kQPrepGroup;
  __shared__ float q[HG][D];
  __shared__ float part[HG][4][64];
  __shared__ float vals[HG][64];
  __shared__ uint2 fx[HG][4][2][32];
  __shared__ int ex[HG][4][2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = blockIdx.x / NSL, t = blockIdx.x % NSL;
  const bool sgn = t >= D / 64;
  const int c0 = (sgn ? t - D / 64 : t) * 64;
  const float *mt = (sgn ? a.projT : a.rotT) + c0 + lane + size_t(wave) * KPT * D;
  float m[KPT];
#pragma unroll
  for (int i = 0; i < KPT; ++i) m[i] = mt[size_t(i) * D];
  for (int i = tid; i < HG * D; i += 256) {
    const int h = i / D, j = i % D, bh = grp * HG + h;
    q[h][j] = bh < nq ? load_q(a.q, a.dtype, size_t(bh) * D + j) : 0.0f;
  }
  __syncthreads();
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
  __syncthreads();
  const int npk = n_walsh(a.k.bq), nplane = sgn ? 1 : npk, ni = q_items<G>(a, sgn);
  for (int e = tid; e < HG * nplane * 64; e += 256) {  // whole waves: the per-word maxima stay in a wave
    const int h = e / (nplane * 64);
    query_fixed_point(a, vals[h], sgn, e % (nplane * 64), fx[h], ex[h], lane);
  }
  __syncthreads();
  for (int e = tid; e < HG * ni; e += 256) {
    const int h = e / ni, bh = grp * HG + h;
    if (bh >= nq) continue;
    const int b = bh / a.Hq, hq = bh % a.Hq;
    pack_query_operand<D, G>(a, fx[h], ex[h], c0, sgn, npk, b * a.Hkv + hq / G, hq % G, e % ni);
  }
}

// ------------------------------------------------------------ split pass ---
// One 256-thread block per (split, kv head, sequence); a split holds at most
// kMaxT * 256 slots.  BQK / BQV: index bits of keys / values (compile time: the
// plane loops unroll without branches); the sign planes always run, with zero
// operands when a tensor has no sketch.
//
// Lane roles: lane = 16 grp + col.  In a score product col is the token of a
// 16-token block and grp the lane group of the contraction (coordinates); the
// result gives lane (col, grp) the digit-slot sums of query heads 4 rb + grp
// (rb < RB) for that token.  In a value MFMA col is the coordinate of a
// 16-coordinate block and grp the token group of the contraction.
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
constexpr int kMaxT = 5;   // key tiles per wave and split: split <= 1280 slots

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
// of it are complete (lgkmcnt(0) first).  NT: a non-temporal load, for data
// that the launch reads once (attention streams each cache line once, and the
// stream then displaces less of what is still to be read, such as the split
// partials the merge reads next).  Key scoring reads the same keys from every
// query group's blocks, and the Sparse V maxima pass reads keys that attention
// reads again: both keep ordinary loads.
template <bool NT>
__device__ inline void dma16(u4 r, unsigned dst, int voff, int soff) {
  if (NT) asm volatile("buffer_load_dwordx4 %0, %1, %2 offen nt lds" ::"v"(voff), "s"(r), "s"(soff), "{m0}"(dst) : "memory");
  else asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(r), "s"(soff), "{m0}"(dst) : "memory");
}
template <bool NT>
__device__ inline void dma4(u4 r, unsigned dst, int voff, int soff) {
  if (NT) asm volatile("buffer_load_dword %0, %1, %2 offen nt lds" ::"v"(voff), "s"(r), "s"(soff), "{m0}"(dst) : "memory");
  else asm volatile("buffer_load_dword %0, %1, %2 offen lds" ::"v"(voff), "s"(r), "s"(soff), "{m0}"(dst) : "memory");
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

template <int D, int RB, int BQK, int BQV, int SLOTS_, int AWP_>
struct SplitShape {
  static constexpr int W = D / 32, NB = D / 64, NW = D / 128, G = 4 * RB;
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
  // Ring slots per wave (SLOTS - 1 chunks in flight) and value operand buffers
  // (AWP = 2: one per round parity, so a round's operands are written while the
  // previous round's are still read).
  static constexpr int SLOTS = SLOTS_;
  static constexpr int AWP = AWP_;
};

// Modes of the split pass:
//   kAttend  attention partials (phase 1 scores, phase 2 values);
//   kScores  key scoring (tq_score_keys): phase 1 only, over key head
//            a.kv_fixed, writing each score instead of a partial;
//   kMaxima  phase 1 only, writing each head's largest score of the split (the
//            first pass of Sparse V decode).
// SPARSE (kAttend only): the value sum leaves out positions whose score is below
// the head's largest score over every split (from a kMaxima pass) plus
// a.sparse_thr = log2(tau), and skips the value products of tiles where that
// leaves nothing; the softmax sum keeps every position.
constexpr int kAttend = 0, kScores = 1, kMaxima = 2;

template <int D, int RB, int BQK, int BQV, int SLOTS, int AWP_, int MODE = kAttend, bool SPARSE = false>
__global__ __launch_bounds__(256) void decode_partial_fast(DecodeArgs a) {
  // non-temporal loads where this pass is the last to read the stream: attention
  // (not the Sparse V maxima pass, whose keys the attention pass reads again)
  constexpr bool SCORES = MODE == kScores, KEYS_ONLY = MODE != kAttend, NT = MODE == kAttend;
  using P = SplitShape<D, RB, BQK, BQV, SLOTS, AWP_>;
  constexpr int W = P::W, NB = P::NB, NW = P::NW, G = P::G, PK = P::PK, PV = P::PV;
  constexpr int KREC = P::KREC, KSREC = P::KSREC, VREC = P::VREC, VSREC = P::VSREC, AWP = P::AWP;
  constexpr int kSlots = P::SLOTS;
  __shared__ __attribute__((aligned(16))) unsigned char ring[4][kSlots][P::SLOT];
  // value A operands of a round: [round parity][part][tile][kgroup][rb][row][byte]
  __shared__ __attribute__((aligned(16))) unsigned char aw[AWP][2][4][4][RB][16][16];
  __shared__ float redf[4][G];
  __shared__ float redv[4][2];
  __shared__ int tflag[AWP][4];  // Sparse V: 1 if tile (round parity, wave) keeps any value
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
  constexpr int stride = part_stride<D>();
  if (lo >= hi) {
    if (MODE == kAttend && tid < G) {
      float *o = a.part + (size_t(bh0 + tid) * a.n_split + split) * stride;
      o[0] = -INFINITY;
      o[1] = 0.0f;
    }
    if (MODE == kMaxima && tid < G) a.smax[size_t(bh0 + tid) * a.n_split + split] = -INFINITY;
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
  const u4 rvc = KEYS_ONLY ? make_rsrc(a.k.scl, 0) : make_rsrc(a.v.scl + (int64_t(h) * vcap + abase) * 2, vslots * 4);
  const u4 rv = KEYS_ONLY ? make_rsrc(a.k.idx, 0) : make_rsrc(a.v.idx + (int64_t(h) * vblocks + blk0) * BQV * D, vblk * VREC);
  const u4 rvs = KEYS_ONLY || !skv ? make_rsrc(a.k.idx, 0) : make_rsrc(a.v.sgn + (int64_t(h) * vblocks + blk0) * D, vblk * VSREC);

  // ---- the wave's chunk stream ----
  const int nk = ntile > wave ? (ntile - wave + 3) >> 2 : 0;  // key tiles of this wave
  const int nr = KEYS_ONLY ? 0 : (ntile + 3) >> 2;            // value rounds
  const int nch = nk + nr;
  // value chunk lane roles: lane -> (block, 16-byte piece) of the wave's coordinates
  const int vblkl = NW == 1 ? (lane >> 3) : (lane >> 4), vpiece = NW == 1 ? (lane & 7) : (lane & 15);
  auto issue = [&](int s) {
    const unsigned dst = lds_addr(&ring[wave][s % kSlots][0]);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (s < nk) {
      const int tile = wave + 4 * s;
#pragma unroll
      for (int i = 0; i < BQK * NW; ++i) dma16<NT>(rk, dst + 1024 * i, tile * 64 * KREC + 1024 * i + 16 * lane, 0);
#pragma unroll
      for (int i = 0; i < NW; ++i) dma16<NT>(rks, dst + P::K_SG + 1024 * i, tile * 64 * KSREC + 1024 * i + 16 * lane, 0);
      dma4<NT>(rkc, dst + P::K_KS, tile * 256 + 4 * lane, 0);
      dma4<NT>(rvc, dst + P::K_VS, tile * 256 + 4 * lane, 0);
    } else {
      const int r = s - nk;
#pragma unroll
      for (int p = 0; p <= BQV; ++p)
#pragma unroll
        for (int i = 0; i < NW; ++i) {
          const bool sg = p == BQV;
          const int rec = sg ? VSREC : VREC;
          const int voff = (8 * r + 4 * i + vblkl) * rec + (sg ? 0 : p * D * 4) + wave * D + 16 * vpiece;
          dma16<NT>(sg ? rvs : rv, dst + p * P::VPL + 1024 * i, voff, 0);
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
  // Query operands of the score products (fp6 digits, six words per lane) and
  // their scale bytes, byte q = (plane (PK: sign) * NW + chunk) * NM + product.
  constexpr int QS = 16 / G, NM = (kQDigits + QS - 1) / QS, NQB = (PK + 1) * NW * NM, NQW = (NQB + 3) / 4;
  uint32_t qa[PK + 1][NW][NM][6];
  uint32_t qsc[NQW];
  {
    const uint32_t *qop = a.qop + size_t(b * a.Hkv + h) * 5 * NW * NM * kWave * 8;
#pragma unroll
    for (int p = 0; p <= PK; ++p) {
      const int slot = p == PK ? kSigPlane : p;
#pragma unroll
      for (int c = 0; c < NW; ++c)
#pragma unroll
        for (int i = 0; i < NM; ++i) {
          const uint32_t *src = qop + (((size_t(slot) * NW + c) * NM + i) * kWave + lane) * 8;
          const uint4 x = *reinterpret_cast<const uint4 *>(src);
          const uint2 y = *reinterpret_cast<const uint2 *>(src + 4);
          qa[p][c][i][0] = x.x;
          qa[p][c][i][1] = x.y;
          qa[p][c][i][2] = x.z;
          qa[p][c][i][3] = x.w;
          qa[p][c][i][4] = y.x;
          qa[p][c][i][5] = y.y;
        }
    }
    const uint32_t *qs = reinterpret_cast<const uint32_t *>(a.qscale + (size_t(b * a.Hkv + h) * kWave + lane) * 32);
#pragma unroll
    for (int k = 0; k < NQW; ++k) qsc[k] = qs[k];
#pragma unroll
    for (int p = 0; p <= PK; ++p)
#pragma unroll
      for (int c = 0; c < NW; ++c)
#pragma unroll
        for (int i = 0; i < NM; ++i)
#pragma unroll
          for (int k = 0; k < 6; ++k) asm volatile("" ::"v"(qa[p][c][i][k]));
#pragma unroll
    for (int k = 0; k < NQW; ++k) asm volatile("" ::"v"(qsc[k]));
  }
  // value products: bit-plane operand bytes (bit << k) and the all-ones plane
  const uint32_t msk[4] = {0x01010101u, 0x02020202u, 0x04040404u, 0x08080808u};
  const v4i ones = {static_cast<int>(msk[0]), static_cast<int>(msk[1]), static_cast<int>(msk[2]),
                    static_cast<int>(msk[3])};
  // The products sum T b over a plane, with T = 2 w v / f and the bit's fp4 value
  // f, i.e. 2 sum_j w v_j b_j.  The +-1 form needs minus sum_j w v_j, half the
  // operand's product with all-ones planes (B = the four masks themselves),
  // which starts every score accumulator, row by row.
  v4f nki = {0.0f, 0.0f, 0.0f, 0.0f}, nks = {0.0f, 0.0f, 0.0f, 0.0f};
  {
    const v8i all = fp4_planes(0xFFFFFFFFu);
#pragma unroll
    for (int c = 0; c < NW; ++c) {
#pragma unroll
      for (int p = 0; p < PK; ++p)
#pragma unroll
        for (int i = 0; i < NM; ++i) nki = qmfma(qa[p][c][i], all, nki, qsc, (p * NW + c) * NM + i);
#pragma unroll
      for (int i = 0; i < NM; ++i) nks = qmfma(qa[PK][c][i], all, nks, qsc, (PK * NW + c) * NM + i);
    }
    nki *= -0.5f;
    nks *= -0.5f;
  }

  // ---- phase 1: scores of this wave's key tiles, kept in registers ----
  float sreg[kMaxT][4][RB];
  uint32_t vreg[kMaxT][4];  // value scales of the same tokens (0 outside the range), for phase 2
  float mloc[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) mloc[rb] = -INFINITY;
  // largest value scales of the split: the fp16 pair (nu~, rho~) as bits, maxima
  // per half (non-negative halves order as unsigned integers)
  us2 vsmax = {0, 0};
  const int nvalid = vhi - vlo;
#pragma unroll
  for (int kt = 0; kt < kMaxT; ++kt) {
    if (kt < nk) {
      issue(kt + kSlots - 1);
      wait_chunk(kt);
      const unsigned char *sl = &ring[wave][kt % kSlots][0];
      const int tile = wave + 4 * kt;
      // Token of lane column col in block nb.  Attention: token 32 (g / 2) + 8 nb + s + 4 (g % 2)
      // with (g, s) = (col / 4, col % 4), the slot that lands in byte nb of operand
      // word s of lane group g of the value products, so that phase 2 can turn
      // the lane's four weights into its operand words in registers.  Scoring:
      // token 16 nb + col, so that a lane group's stores are 16 consecutive scores.
      const int tok0 = SCORES ? col : 32 * (col >> 3) + 4 * ((col >> 2) & 1) + (col & 3);
      const int tstep = SCORES ? 16 : 8;
      const int rel = tile * 64 + tok0 - vlo;  // slot of the lane's token of block 0, from the first valid one
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int tok = tok0 + tstep * nb, t = tile * 64 + tok;
        const bool valid = static_cast<unsigned>(rel + tstep * nb) < static_cast<unsigned>(nvalid);
        // lane group grp holds words grp, grp + 4, ... of the token's planes
        uint32_t wd[3][NW], ws[NW];
#pragma unroll
        for (int u = 0; u < NW; ++u) {
#pragma unroll
          for (int p = 0; p < 3; ++p) wd[p][u] = p < BQK ? lds32(sl + tok * KREC + p * W * 4 + (grp + 4 * u) * 4) : 0u;
          ws[u] = lds32(sl + P::K_SG + tok * KSREC + (grp + 4 * u) * 4);
        }
        const uint32_t ksc = lds32(sl + P::K_KS + 4 * tok), vsc = lds32(sl + P::K_VS + 4 * tok);
        v4f acc_i = nki, acc_s = nks;
#pragma unroll
        for (int c = 0; c < NW; ++c) {
#pragma unroll
          for (int p = 0; p < PK; ++p) {
            const v8i B = fp4_planes(plane_word<4>(p, wd[0][c], wd[1][c], wd[2][c]));
#pragma unroll
            for (int i = 0; i < NM; ++i) acc_i = qmfma(qa[p][c][i], B, acc_i, qsc, (p * NW + c) * NM + i);
          }
          const v8i B = fp4_planes(ws[c]);
#pragma unroll
          for (int i = 0; i < NM; ++i) acc_s = qmfma(qa[PK][c][i], B, acc_s, qsc, (PK * NW + c) * NM + i);
        }
        const float knu = f16v(ksc), krho = f16v(ksc >> 16);
        const uint32_t vscv = valid ? vsc : 0u;
        vreg[kt][nb] = vscv;
        vsmax = __builtin_elementwise_max(vsmax, __builtin_bit_cast(us2, vscv));
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          // rows QS rb .. QS rb + QS - 1 of this lane: the digit slots of head 4 rb + grp
          float ri = acc_i[QS * rb], rs = acc_s[QS * rb];
#pragma unroll
          for (int u = 1; u < QS; ++u) {
            ri += acc_i[QS * rb + u];
            rs += acc_s[QS * rb + u];
          }
          float sv = fmaf(knu, ri, krho * rs);
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
  if (MODE == kMaxima) {
    if (col == 0)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) redf[wave][rb * 4 + grp] = mloc[rb];
    wait_vm<0>();
    lds_barrier();
    if (tid < G)
      a.smax[size_t(bh0 + tid) * a.n_split + split] =
          fmaxf(fmaxf(redf[0][tid], redf[1][tid]), fmaxf(redf[2][tid], redf[3][tid]));
    return;
  }
  float vnumax = f16v(vsmax.x), vrhomax = f16v(vsmax.y);
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
  // Sparse V: the value of a position is kept when its score reaches the head's
  // largest score over every split plus log2(tau)
  float thr[RB];
  if constexpr (SPARSE) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float *sm = a.smax + size_t(bh0 + rb * 4 + grp) * a.n_split;
      float m = -INFINITY;
      for (int sp = col; sp < a.n_split; sp += 16) m = fmaxf(m, sm[sp]);
#pragma unroll
      for (int o = 8; o > 0; o >>= 1) m = fmaxf(m, lane_xor_f(m, o, lane));
      thr[rb] = m + a.sparse_thr;
    }
  }

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
        // Weights of this wave's tile 4 r + wave (its key tile r).  Lane (col, grp)
        // holds the scores of head 4 rb + grp for its four tokens (blocks nb), which
        // are bytes nb of operand word s = col % 4 of lane group g = col / 4 of the
        // value products.  Each weight becomes the four signed digits of its
        // fixed-point value (weight, then residual weight); a 4 x 4 byte transpose
        // gives, per digit l, the word of row (head grp, digit l) at word s of lane
        // group g.  Rows are stored XOR-swizzled by g (row ^ g), so that the 64
        // lanes' stores fall in distinct banks.  A token outside the range has
        // score -inf (weight 0) and value scales 0.
        const float s2 = ldexpf(1.0f, Ew - (col & 3)), s2p = ldexpf(1.0f, Ewp - (col & 3));
        uint32_t dw[2][RB][4];
        bool keep_any = false;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const float vnu = f16v(vreg[r][nb]), vrho = f16v(vreg[r][nb] >> 16);
          const float sw = vnu * s2, swp = vrho * s2p;  // scale 2^(E - s), exact
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            const float Pw = __builtin_amdgcn_exp2f(sreg[r][nb][rb] - mh[rb]);
            lloc[rb] += Pw;
            float Pv = Pw;  // the weight of the position's value
            if constexpr (SPARSE) {
              Pv = sreg[r][nb][rb] >= thr[rb] ? Pw : 0.0f;
              keep_any |= Pv > 0.0f;
            }
            // truncation toward zero: |error| < 1 unit of 2^-Ew, far below the
            // 24-bit resolution of the float weight itself
            dw[0][rb][nb] = digits(static_cast<int32_t>(Pv * sw));
            dw[1][rb][nb] = digits(static_cast<int32_t>(Pv * swp));
          }
        }
        if constexpr (SPARSE) {
          const bool any = __ballot(keep_any) != 0;
          if (lane == 0) tflag[par][wave] = any;
        }
        const int g = col >> 2, sw4 = 4 * (col & 3);
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            const uint32_t *a4 = dw[x][rb];
            const uint32_t t0 = __builtin_amdgcn_perm(a4[1], a4[0], 0x05010400u);  // a0.d0 a1.d0 a0.d1 a1.d1
            const uint32_t t1 = __builtin_amdgcn_perm(a4[1], a4[0], 0x07030602u);  // a0.d2 a1.d2 a0.d3 a1.d3
            const uint32_t t2 = __builtin_amdgcn_perm(a4[3], a4[2], 0x05010400u);
            const uint32_t t3 = __builtin_amdgcn_perm(a4[3], a4[2], 0x07030602u);
            const uint32_t o[4] = {__builtin_amdgcn_perm(t2, t0, 0x05040100u), __builtin_amdgcn_perm(t2, t0, 0x07060302u),
                                   __builtin_amdgcn_perm(t3, t1, 0x05040100u), __builtin_amdgcn_perm(t3, t1, 0x07060302u)};
#pragma unroll
            for (int l = 0; l < 4; ++l)
              *reinterpret_cast<uint32_t *>(&aw[par][x][wave][g][rb][(4 * grp + l) ^ g][sw4]) = o[l];
          }
      }
      lds_barrier();
      wait_chunk(s);
      const unsigned char *sl = &ring[wave][s % kSlots][0];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        if (4 * r + tt >= ntile) break;
        if (SPARSE && !tflag[par][tt]) continue;  // every value of the tile is left out
        v4i aw0[RB], aw1[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          aw0[rb] = *reinterpret_cast<const v4i *>(&aw[par][0][tt][grp][rb][col ^ grp][0]);
          aw1[rb] = *reinterpret_cast<const v4i *>(&aw[par][1][tt][grp][rb][col ^ grp][0]);
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
      o[4 + j0 + nb] = static_cast<float>(ldexp(acc, -Ew));
      o[4 + D + j0 + nb] = skv ? static_cast<float>(ldexp(pm_form(av[PV][nb][rb], ak[1][rb]), -Ewp)) : 0.0f;
    }
    if (wave == 0 && col == 0) {
      o[0] = mh[rb] * 0.69314718055994531f;  // natural-log units for the merge
      o[1] = lh_s[head];
    }
  }
}

// ----------------------------------------------------------------- merge ---
// out = (Pi^T A + kappa S^T B) / l, where (A, B) and l merge the split partials
// by log-sum-exp.  A partial record is m, l, two pad words, A [d], B [d]
// (kPartStride floats, so that (A, B) start 16-byte aligned).  Block (head, cs)
// computes the CPB x 64 outputs from 64 CPB cs on (CPB = d / 64, one block per
// head, when there are heads enough to fill the chip; else CPB = 1):
//  1. the split maxima and sums: M = max m_s over splits with tokens, weights
//     w_s = exp(m_s - M) (0 for a split with no tokens, whose (A, B) are
//     unwritten), l = sum w_s l_s; the weights go to LDS.
//  2. thread (sg, c) sums w_s x_s for the 16-byte chunk c of (A, B) over splits
//     sg, sg + SGN, ...; its loads are issued before step 1 (they do not depend
//     on the weights), as are the matrix loads of step 3.  The split groups are
//     added in LDS, kappa B formed there.
//  3. per group of 64 columns, thread (kq, jj) takes entries kq 2d/8 ..
//     (kq + 1) 2d/8 - 1 of [A ; kappa B] against the matching row segment of
//     Pi^T (rows of A) or S^T (rows of B), both read as 16-byte chunks of the
//     transposed matrices; the 8 partial sums are added in LDS.
// Every block of a head recomputes steps 1-2 so that no block waits on another.
constexpr int kMaxSplits = 2048;

template <int D, int CPB>
__global__ __launch_bounds__(512) void decode_merge_fast(DecodeArgs a) {
  constexpr int NT = 512, NC4 = 2 * D / 4, SGN = NT / NC4;  // chunks of (A, B), split groups
  constexpr int CHS = D == 128 ? 16 : 20;                      // split loads per thread and round
  constexpr int KR = 2 * D / 8, KR4 = KR / 4;                 // step 3: entries per thread
  constexpr int stride = part_stride<D>();
  __shared__ float ws_l[kMaxSplits], ls_l[kMaxSplits];
  __shared__ float red[8];
  __shared__ __attribute__((aligned(16))) float4 accg[SGN][NC4];
  __shared__ __attribute__((aligned(16))) float vec[2 * D];
  __shared__ float prj[8][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int ncs = D / (64 * CPB);
  const int bh = blockIdx.x / ncs, cs = blockIdx.x % ncs;
  const int ns = a.n_split;
  const float *base = a.part + size_t(bh) * ns * stride;
  // step 3's matrix rows: column col of the output = row col of Pi^T / S^T,
  // entries kq KR .. kq KR + KR - 1 of [A ; B] (kq < 4: Pi^T; else S^T)
  const int jj = tid & 63, kq = tid >> 6;
  const float *mt = kq < 4 ? a.rotT : a.projT;
  const int k0 = (kq & 3) * KR;
  float4 mrow[KR4];
  auto load_rows = [&](int col) {
#pragma unroll
    for (int i = 0; i < KR4; ++i) mrow[i] = *reinterpret_cast<const float4 *>(mt + size_t(col) * D + k0 + 4 * i);
  };
  load_rows(64 * CPB * cs + jj);
  // step 2's first round of loads
  const int c4 = tid % NC4, sg = tid / NC4;
  float4 x[CHS];
  auto load_x = [&](int s0) {
#pragma unroll
    for (int u = 0; u < CHS; ++u) {
      const int sp = s0 + sg + SGN * u;
      x[u] = sp < ns ? *reinterpret_cast<const float4 *>(base + size_t(sp) * stride + 4 + 4 * c4)
                     : float4{0.0f, 0.0f, 0.0f, 0.0f};
    }
  };
  load_x(0);
  // step 1
  float mmax = -INFINITY;
  for (int sp = tid; sp < ns; sp += NT) {
    const float2 ml = *reinterpret_cast<const float2 *>(base + size_t(sp) * stride);
    ws_l[sp] = ml.y > 0.0f ? ml.x : -INFINITY;
    ls_l[sp] = ml.y > 0.0f ? ml.y : 0.0f;
    mmax = fmaxf(mmax, ws_l[sp]);
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
  for (int sp = tid; sp < ns; sp += NT) {
    const float ms = ws_l[sp];
    const float w = ms > -INFINITY ? expf(ms - M) : 0.0f;
    lsum = fmaf(w, ls_l[sp], lsum);
    ws_l[sp] = w;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) lsum += lane_xor_f(lsum, o, lane);
  if (lane == 0) red[wave] = lsum;
  __syncthreads();
  float l = 0.0f;
#pragma unroll
  for (int w = 0; w < 8; ++w) l += red[w];
  // step 2
  float4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int s0 = 0; s0 < ns; s0 += SGN * CHS) {
    if (s0 > 0) load_x(s0);
#pragma unroll
    for (int u = 0; u < CHS; ++u) {
      const int sp = s0 + sg + SGN * u;
      const float w = sp < ns ? ws_l[sp] : 0.0f;
      if (w > 0.0f) {  // a split without tokens has stale (A, B)
        acc.x = fmaf(w, x[u].x, acc.x);
        acc.y = fmaf(w, x[u].y, acc.y);
        acc.z = fmaf(w, x[u].z, acc.z);
        acc.w = fmaf(w, x[u].w, acc.w);
      }
    }
  }
  accg[sg][c4] = acc;
  __syncthreads();
  if (tid < 2 * D) {
    const float *ag = reinterpret_cast<const float *>(accg);
    float v = 0.0f;
#pragma unroll
    for (int g = 0; g < SGN; ++g) v += ag[g * 2 * D + tid];
    vec[tid] = tid < D ? v : a.kappa * v;
  }
  __syncthreads();
  // step 3
  float4 vk[KR4];
#pragma unroll
  for (int i = 0; i < KR4; ++i) vk[i] = *reinterpret_cast<const float4 *>(&vec[kq * KR + 4 * i]);
#pragma unroll 1
  for (int cg = 0; cg < CPB; ++cg) {
    if (cg > 0) {
      load_rows(64 * (CPB * cs + cg) + jj);
      __syncthreads();  // prj of the previous group has been read
    }
    float pj = 0.0f;
#pragma unroll
    for (int i = 0; i < KR4; ++i) {
      pj = fmaf(mrow[i].x, vk[i].x, pj);
      pj = fmaf(mrow[i].y, vk[i].y, pj);
      pj = fmaf(mrow[i].z, vk[i].z, pj);
      pj = fmaf(mrow[i].w, vk[i].w, pj);
    }
    prj[kq][jj] = pj;
    __syncthreads();
    if (tid < 64) {
      float o = 0.0f;
#pragma unroll
      for (int g = 0; g < 8; ++g) o += prj[g][tid];
      a.out[size_t(bh) * D + 64 * (CPB * cs + cg) + tid] = l > 0.0f ? o / l : 0.0f;
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
  constexpr int stride = part_stride<D>();
  const int ns = a.n_split;
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
          // (A, B) start 16 bytes into the record: 16-byte chunks
#pragma unroll
          for (int e = 0; e < EPT; e += 4) {
            const float4 v4 = *reinterpret_cast<const float4 *>(p + 4 + lane * EPT + e);
            x[u][e] = v4.x;
            x[u][e + 1] = v4.y;
            x[u][e + 2] = v4.z;
            x[u][e + 3] = v4.w;
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

template <int D, int RB, int BQK, int SLOTS, int AWP, bool SPARSE>
int launch_partial_bv(int bqv, const DecodeArgs &a, hipStream_t s) {
  const dim3 grid(a.n_split, a.Hkv, a.batch);
  if (a.split_tokens > kMaxT * 256 || a.n_split > kMaxSplits) return 1;
  if (SPARSE)  // first pass: every split's largest score per head
    hipLaunchKernelGGL((decode_partial_fast<D, RB, BQK, BQK, SLOTS, AWP, kMaxima>), grid, dim3(256), 0, s, a);
  switch (bqv) {
    case 1: hipLaunchKernelGGL((decode_partial_fast<D, RB, BQK, 1, SLOTS, AWP, kAttend, SPARSE>), grid, dim3(256), 0, s, a); return 0;
    case 2: hipLaunchKernelGGL((decode_partial_fast<D, RB, BQK, 2, SLOTS, AWP, kAttend, SPARSE>), grid, dim3(256), 0, s, a); return 0;
    case 3: hipLaunchKernelGGL((decode_partial_fast<D, RB, BQK, 3, SLOTS, AWP, kAttend, SPARSE>), grid, dim3(256), 0, s, a); return 0;
    default: return 1;
  }
}

template <int D, int RB, int SLOTS, int AWP, bool SPARSE>
int launch_partial(const DecodeArgs &a, hipStream_t s) {
  switch (a.k.bq) {
    case 1: return launch_partial_bv<D, RB, 1, SLOTS, AWP, SPARSE>(a.v.bq, a, s);
    case 2: return launch_partial_bv<D, RB, 2, SLOTS, AWP, SPARSE>(a.v.bq, a, s);
    case 3: return launch_partial_bv<D, RB, 3, SLOTS, AWP, SPARSE>(a.v.bq, a, s);
    default: return 1;
  }
}

// Query prep: per-head blocks, or groups of kQPrepGroup heads when there are many.
template <int D, int G>
void launch_qprep_g(const DecodeArgs &a, hipStream_t s) {
  const unsigned nq = static_cast<unsigned>(a.batch * a.Hq);
  if (nq >= 512)
    hipLaunchKernelGGL((decode_qprep_grouped<D, G>), dim3((nq + kQPrepGroup - 1) / kQPrepGroup * (2 * D / 64)),
                       dim3(256), 0, s, a, int(nq));
  else hipLaunchKernelGGL((decode_qprep_fast<D, G>), dim3(nq * (2 * D / 64)), dim3(256), 0, s, a);
}

template <int D>
int launch_qprep(const DecodeArgs &a, hipStream_t s) {
  switch (a.G) {
    case 4: launch_qprep_g<D, 4>(a, s); return 0;
    case 8: launch_qprep_g<D, 8>(a, s); return 0;
    case 16: launch_qprep_g<D, 16>(a, s); return 0;
    default: return 1;
  }
}

// Ring depth of the split pass (slots per wave) for one and two row blocks of
// heads when the grid is large, so that several work-groups share a CU.
constexpr int kSlotsRb1 = 2, kSlotsRb2 = 2;

template <int D>
int launch_fast_d(int rb, const DecodeArgs &a, hipStream_t s, bool sparse) {
  const unsigned nq = static_cast<unsigned>(a.batch * a.Hq);
  if (launch_qprep<D>(a, s)) return 1;
  // one head block and at most about two work-groups per CU: a deep ring (two
  // chunks in flight per wave) and two operand buffers
  const bool deep = int64_t(a.n_split) * a.Hkv * a.batch <= 1024;
  int e;
  if (sparse)
    e = rb == 2 ? launch_partial<D, 2, kSlotsRb2, 1, true>(a, s)
                : deep ? launch_partial<D, 1, 3, 2, true>(a, s) : launch_partial<D, 1, kSlotsRb1, 1, true>(a, s);
  else
    e = rb == 2 ? launch_partial<D, 2, kSlotsRb2, 1, false>(a, s)
                : deep ? launch_partial<D, 1, 3, 2, false>(a, s) : launch_partial<D, 1, kSlotsRb1, 1, false>(a, s);
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
  constexpr int SLOTS = DEEP ? 3 : 2, AWP = DEEP ? 2 : 1;
  // splits rounded up to a multiple of 8 (the XCD count); the extra work-groups
  // find an empty range and return
  const dim3 grid((a.n_split + 7) / 8 * 8 * a.Hkv, 1, a.batch);
  if (a.split_tokens > kMaxT * 256) return 1;
  hipLaunchKernelGGL((decode_partial_fast<D, RB, BQK, BQK, SLOTS, AWP, kScores>), grid, dim3(256), 0, s, a);
  return 0;
}

template <int D>
int launch_score_d(const DecodeArgs &a, hipStream_t s) {
  if (launch_qprep<D>(a, s)) return 1;
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

int launch_decode_fast(int d, int rb, const DecodeArgs &a, hipStream_t s, bool sparse) {
  int e = 1;
  if (d == 128) e = launch_fast_d<128>(rb, a, s, sparse);
  else if (d == 256) e = launch_fast_d<256>(rb, a, s, sparse);
  if (e) return e;
  return hipGetLastError() != hipSuccess;
}

}  // namespace tq
