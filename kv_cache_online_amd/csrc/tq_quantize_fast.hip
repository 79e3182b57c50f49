// Matrix-core quantize for d = m = 128 (and, further down, d = m = 256 with
// bf16 input) on gfx950.
//
// Method: ast-softpro.ru, "Технология TurboQuant и её применение с локальными
// LLM", section 1.2 "Как работает TurboQuant" -- stage 1 rotates x by Pi and
// picks a Lloyd-Max cell per coordinate of u = Pi x / ||x||; stage 2 keeps
// sign(S r) and ||r||_2 of the residual r = x - ||x||~ Pi^T c[idx].  As in the
// reference-grade kernel, the residual is formed in the rotated frame,
// rho = Pi x - ||x||~ c[idx], and sketched as S~ rho with S~ = S Pi^T.
//
// Both contractions are dense (a 128 x 128 matrix against a tile of vectors),
// so they run on v_mfma_f32_16x16x32_bf16.  Every operand is split into bf16
// pieces (hi + mid + lo reproduces an fp32 value exactly); the piece products
// are exact in fp32, and the dropped cross terms are below 2^-24 relative for
// Pi x and below 2^-16 relative for the sketch, whose only use is a sign.
//
// Work-group: 4 waves, two work-groups per CU so that one group's matrix
// phase overlaps the other's vector phase; persistent over tiles of 32
// vectors of one (sequence, head).  Tiles are aligned to 32-slot blocks of the
// cache.  Wave w owns rotated coordinates and sketch rows 32w .. 32w+31 and
// keeps those rows of Pi and S~ in registers as the MFMA row operand; the
// tile of vectors is the column operand, so a lane of the result holds four
// consecutive coordinates of one vector.  Per tile:
//   A  load (the next tile is prefetched into registers), ||x||, per-vector
//      boundaries ||x|| t_k and scaled centroids ||x||~ c_k, input -> LDS
//   B  z = Pi x; cells by comparing |z| with ||x|| t_k; the compare masks are
//      the bit planes, one 32-bit word per coordinate over the 32 slots; the
//      residual's bf16 pieces -> LDS; partial ||rho||^2 per wave
//   D  p = S~ rho; sign masks the same way; ||rho|| per vector
//   E  records to HBM: the words are the value layout as they stand; the
//      token-major key layout takes a 32 x 32 bit transpose per word block
// The codebook must be symmetric (c[L-1-i] = -c[i], middle boundary 0), as
// the Lloyd-Max codebook of the symmetric coordinate law is.

#include <hip/hip_runtime.h>

#include <cmath>

#include "tq_common.h"
#include "tq_device.h"

namespace tq {
namespace {

constexpr int QD = 128;      // d = m
constexpr int QT = 32;       // vectors per tile
constexpr int QW = 4;        // waves per work-group
constexpr int QN = 64 * QW;  // threads per work-group
constexpr int XS = QD + 8;   // bf16 row stride of the operand tiles (elements)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

template <int NPX, int BQ>
struct QSmem {
  __align__(16) uint16_t plo[NPX == 1 ? QD : 1][XS];  // lo piece of Pi (bf16 bits; bf16 input only)
  __align__(16) uint16_t xs[NPX][QT][XS];    // input pieces (bf16 bits)
  __align__(16) uint16_t rh[QT][XS];         // residual, hi piece
  __align__(16) uint16_t rm[QT][XS];         // residual, mid piece
  __align__(16) float vth[QT][8];            // per vector: ||x|| t_k at 0..2, ||x||~ c_k at 4..7
  __align__(16) float rr[QW][QT];            // ||rho||^2 over each wave's coordinates
  __align__(16) uint16_t wst[BQ + 1][QD][2]; // words (plane, coordinate), bit = row; plane BQ: signs
  __align__(16) uint32_t nub[QT];            // fp16 bits of ||x||
  __align__(16) uint32_t scl[QT];            // nu bits | rho bits << 16
  int64_t gslot[QT];                          // gather tiles: destination slot per row (-1: none)
  int32_t ghead[QT];                          // gather tiles: head per row
};

struct Tile {
  int b, h;
  int tensor;     // 0: QuantArgs::t, 1: QuantArgs::t2
  uint32_t g0;    // gather tiles: first vector of the flattened [batch][H][n_new] list
  int t0;         // token of row 0 (negative when the tile starts before the first token)
  int64_t base;   // slot of row 0, a multiple of 32
};

// Division by a run-time constant d >= 1 for dividends below 2^31:
// q = (umulhi(n, m) + n) >> s with s = ceil(log2 d), m = 2^32 (2^s - d) / d + 1.
struct FastDiv {
  uint32_t d, m, s;
};

__host__ inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t s = 0;
  while ((uint64_t(1) << s) < d) ++s;
  const uint64_t m = ((uint64_t(1) << 32) * ((uint64_t(1) << s) - d)) / d + 1;
  return FastDiv{d, static_cast<uint32_t>(m), s};
}

__device__ inline uint32_t fdiv(uint32_t n, FastDiv f) { return (__umulhi(n, f.m) + n) >> f.s; }

// A wave-uniform read of memory that no kernel of this launch writes, through
// the scalar cache (constant address space): its wait is on the scalar counter,
// so it does not wait behind the wave's outstanding vector loads and stores.
__device__ inline int64_t load_uniform(const int64_t *p) {
  return *reinterpret_cast<const __attribute__((address_space(4))) int64_t *>(reinterpret_cast<uintptr_t>(p));
}

// Tile `tile` of TT vectors: tiles run over (tensor, sequence, head, k), n1 per
// tensor, and tile k of a sequence starts at the 32-slot boundary at or below its
// first slot, plus TT k.
template <int TT>
__device__ inline Tile tile_at(const QuantArgs &a, uint32_t tile, uint32_t n1, FastDiv ftpb, FastDiv fh) {
  Tile T;
  T.tensor = tile >= n1 ? 1 : 0;
  if (T.tensor) tile -= n1;
  const uint32_t bh = fdiv(tile, ftpb);
  const int k = static_cast<int>(tile - bh * ftpb.d);
  T.b = static_cast<int>(fdiv(bh, fh));
  T.h = static_cast<int>(bh - uint32_t(T.b) * fh.d);
  const int64_t d0 = load_uniform(a.dst + T.b);
  const int sh = static_cast<int>(d0 & 31);
  T.base = (d0 - sh) + TT * int64_t(k);
  T.t0 = TT * k - sh;
  return T;
}

// Gather tiles, for appends of a few tokens per sequence: tile k of a tensor holds
// vectors 32 k .. 32 k + 31 of the flattened [batch][H][n_new] list, whatever
// their sequences and heads, so that no matrix work goes to empty rows.
__device__ inline Tile gather_tile_at(uint32_t tile, uint32_t n1) {
  Tile T{};
  T.tensor = tile >= n1 ? 1 : 0;
  T.g0 = (T.tensor ? tile - n1 : tile) * QT;
  return T;
}

// Row v of a tile: whether it holds a vector, that vector's index in the input
// ([batch][H][n_new] flattened), its head and its destination slot.  fn divides
// by n_new (gather tiles only).
struct Row {
  bool valid;
  size_t i;
  int h;
  int64_t slot;
};

template <bool GATHER>
__device__ inline Row row_at(const QuantArgs &a, const Tile &T, int v, FastDiv fn, FastDiv fh) {
  Row r;
  if (GATHER) {
    // the flattened list holds fewer than 2^31 vectors (checked at launch)
    const uint32_t n = uint32_t(a.batch) * uint32_t(a.H) * uint32_t(a.n_new);
    const uint32_t i = T.g0 + v;
    r.valid = i < n;
    const uint32_t ic = r.valid ? i : 0u;  // every read stays inside dst
    const uint32_t bh = fdiv(ic, fn);
    const uint32_t b = fdiv(bh, fh);
    r.i = ic;
    r.h = static_cast<int>(bh - b * fh.d);
    r.slot = a.dst[b] + int64_t(ic - bh * fn.d);
  } else {
    const int tok = T.t0 + v;
    r.valid = tok >= 0 && tok < a.n_new;
    r.i = (size_t(T.b) * a.H + T.h) * size_t(a.n_new) + tok;
    r.h = T.h;
    r.slot = T.base + v;
  }
  return r;
}

// Row v, coordinates 16 c16 .. 16 c16 + 15 of a tile (zeros outside the tokens).
template <bool F32, bool GATHER>
__device__ inline void load_rows(const QuantArgs &a, const Tile &T, int v, int c16, uint4 *r, FastDiv fn,
                                 FastDiv fh) {
  constexpr int NV = F32 ? 4 : 2;
  const Row rw = row_at<GATHER>(a, T, v, fn, fh);
  if (rw.valid) {
    const size_t row = rw.i;
    const void *x = T.tensor ? a.t2.x : a.t.x;
    const uint4 *p = F32 ? reinterpret_cast<const uint4 *>(static_cast<const float *>(x) + row * QD + 16 * c16)
                         : reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(x) + row * QD + 16 * c16);
#pragma unroll
    for (int i = 0; i < NV; ++i) r[i] = p[i];
  } else {
#pragma unroll
    for (int i = 0; i < NV; ++i) r[i] = make_uint4(0, 0, 0, 0);
  }
}

// IEEE binary16 bits of v >= 0 by the hardware conversion (round to nearest
// even); v > 65504 saturates to 65504 and sets *over.  Rounding a float64
// value through float32 first can differ from a direct rounding only within
// 2^-24 relative of an fp16 rounding midpoint.
__device__ inline uint32_t f16_bits_f32(float v, bool *over) {
  if (!(v == v)) return 0x7E00u;
  if (v > 65504.0f) {
    *over = true;
    return 0x7BFFu;
  }
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(v));
}

__device__ inline uint32_t cvt_pk_bf16(float a, float b) {
  const f32x2 p = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(p, bf16x2));
}

// v_writelane_b32 through the compiler's own intrinsic (this clang has no
// builtin for it), so that its hazard handling sees the instruction: a
// writelane that reads a compare mask needs wait states after the v_cmp.
extern "C" __device__ int tq_writelane_i32(int v, int lane, int old) __asm("llvm.amdgcn.writelane.i32");

// Lane `lane` of `old` takes the wave-uniform value v (EXEC is ignored).
__device__ inline uint32_t wlane(uint32_t v, int lane, uint32_t old) {
  return static_cast<uint32_t>(tq_writelane_i32(static_cast<int>(v), lane, static_cast<int>(old)));
}

// Sum of v over the lanes of an aligned group of 2^k lanes (k <= 3), in every
// lane of the group, by DPP exchanges (lane_xor).
template <int K>
__device__ inline float group_sum(float v, int lane) {
#pragma unroll
  for (int s = 1 << (K - 1); s > 0; s >>= 1)
    v += __uint_as_float(lane_xor(__float_as_uint(v), s, lane));
  return v;
}

// Transpose a 32 x 32 bit matrix held one row per lane (lanes 0-31 and 32-63
// each hold one matrix): afterwards bit c of lane l is bit l of row c.  Step
// s exchanges s-bit blocks with lane row ^ s; both candidates are formed and
// selected, so no step branches.
__device__ inline uint32_t transpose32(uint32_t a, int row) {
  const uint32_t lo_mask[5] = {0x0000FFFFu, 0x00FF00FFu, 0x0F0F0F0Fu, 0x33333333u, 0x55555555u};
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const int s = 16 >> i;
    const uint32_t m = lo_mask[i];
    const uint32_t p = lane_xor(a, s, row);
    const bool hi = (row & s) != 0;
    const uint32_t x = hi ? (p >> s) : (p << s);  // the partner's block, moved into place
    const uint32_t keep = hi ? ~m : m;             // this lane's own bits
    a = (a & keep) | (x & ~keep);
  }
  return a;
}

// The 16 compare masks of one plane (2 row blocks x 2 column groups x 4
// registers), gathered into lanes 0..31 of a VGPR and stored as half-words of
// the (plane, coordinate) words: lane (rb 16 + r 4 + g2 2 + hh) holds mask
// dword hh, whose low half is coordinate 16 rb + 8 hh + r (vectors 16 g2 ..
// 16 g2 + 15) and whose high half is that coordinate + 4.
struct PlaneBits {
  uint32_t pk = 0;
  __device__ inline void put(uint64_t m, int rb, int g2, int r) {
    const int l = rb * 16 + r * 4 + g2 * 2;
    pk = wlane(static_cast<uint32_t>(m), l, pk);
    pk = wlane(static_cast<uint32_t>(m >> 32), l + 1, pk);
  }
  __device__ inline void store(uint16_t (*w)[2], int lane, int c0) const {
    if (lane < 32) {
      const int rb = lane >> 4, r = (lane >> 2) & 3, g2 = (lane >> 1) & 1, hh = lane & 1;
      const int c = c0 + 16 * rb + 8 * hh + r;
      w[c][g2] = static_cast<uint16_t>(pk);
      w[c + 4][g2] = static_cast<uint16_t>(pk >> 16);
    }
  }
};

// GATHER: tiles of the flattened vector list (ftpb then divides by n_new).
template <int BQ, bool F32, bool GATHER>
__global__ __launch_bounds__(QN, 2) void quantize_mfma(QuantArgs a, uint32_t n_tiles, uint32_t n1, FastDiv ftpb, FastDiv fh) {
  constexpr int NPX = F32 ? 3 : 1;
  constexpr int NV = F32 ? 4 : 2;
  constexpr int L = 1 << BQ;
  constexpr int K = L / 2 - 1;  // positive boundaries
  __shared__ QSmem<NPX, BQ> sm;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, li = lane & 15, lg = lane >> 4;
  const int v = t >> 3, c16 = t & 7;  // phase A: row v, coordinates 16 c16 .. 16 c16 + 15
  const int cw = 32 * w;              // first coordinate / sketch row of this wave
  const bool sk = a.t.sketch != 0;

  // Row operands: rows cw + 16 rb + li of Pi and S~, 8 consecutive columns per lane group.
  // The wave's rows of Pi and S~ in registers.  For bf16 input the lo piece of Pi
  // (whose products are 2^-16 of the total) is read from LDS instead, which frees
  // the registers that let a row block's compares overlap the next block's
  // products; fp32 input needs the LDS for its own three pieces.
  constexpr int NPI = F32 ? 3 : 2;
  bf16x8 pia[NPI][2][4], sta[2][2][4];
  if (!F32)
    for (int i = t; i < QD * QD / 8; i += QN) {
      const int r = i / (QD / 8), c8 = i % (QD / 8);
      *reinterpret_cast<uint4 *>(&sm.plo[r][8 * c8]) =
          *reinterpret_cast<const uint4 *>(a.rot_hml + (size_t(2) * QD + r) * QD + 8 * c8);
    }
#pragma unroll
  for (int p = 0; p < NPI; ++p)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int kc = 0; kc < 4; ++kc)
        pia[p][rb][kc] = *reinterpret_cast<const bf16x8 *>(a.rot_hml + (size_t(p) * QD + cw + 16 * rb + li) * QD +
                                                            32 * kc + 8 * lg);
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int kc = 0; kc < 4; ++kc)
        sta[p][rb][kc] = sk ? *reinterpret_cast<const bf16x8 *>(a.st_hml + (size_t(p) * QD + cw + 16 * rb + li) * QD +
                                                                 32 * kc + 8 * lg)
                            : bf16x8{};

  // this lane's coefficient of its vth entry (phase A): upper-half boundary
  // c16 (c16 < K) or centroid c16 - 4 (4 <= c16 <= 4 + K), else 0
  float vcoef = 0.0f;
#pragma unroll
  for (int k = 0; k < K; ++k) vcoef = c16 == k ? a.t.cb.thr[L / 2 + k] : vcoef;
#pragma unroll
  for (int k = 0; k <= K; ++k) vcoef = c16 == 4 + k ? a.t.cb.cen[L / 2 + k] : vcoef;

  uint32_t flags = 0;
  uint4 xr[NV];
  uint32_t tile = blockIdx.x;
  Tile T{};
  auto tile_of = [&](uint32_t k) { return GATHER ? gather_tile_at(k, n1) : tile_at<QT>(a, k, n1, ftpb, fh); };
  if (tile < n_tiles) {
    T = tile_of(tile);
    load_rows<F32, GATHER>(a, T, v, c16, xr, ftpb, fh);
  }
  for (; tile < n_tiles; tile += gridDim.x) {
    const Tile cur = T;
    const QuantTensorArgs &tt = cur.tensor ? a.t2 : a.t;  // this tile's tensor
    uint4 xc[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) xc[i] = xr[i];
    const uint32_t nxt = tile + gridDim.x;
    if (nxt < n_tiles) {
      T = tile_of(nxt);
      load_rows<F32, GATHER>(a, T, v, c16, xr, ftpb, fh);
    }
    // no token falls in this tile (uniform)
    if (GATHER ? cur.g0 >= uint32_t(a.batch) * uint32_t(a.H) * uint32_t(a.n_new) : cur.t0 >= a.n_new) continue;

    // ---------------------------------------------------------------- A --
    {
      const uint32_t *u = reinterpret_cast<const uint32_t *>(xc);
      float ssf = 0.0f;
      if (F32) {
#pragma unroll
        for (int i = 0; i < 16; ++i) ssf = fmaf(__uint_as_float(u[i]), __uint_as_float(u[i]), ssf);
        uint32_t pc[3][8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float x0 = __uint_as_float(u[2 * i]), x1 = __uint_as_float(u[2 * i + 1]);
          const uint32_t h = cvt_pk_bf16(x0, x1);
          const float r0 = x0 - __uint_as_float(h << 16), r1 = x1 - __uint_as_float(h & 0xFFFF0000u);
          const uint32_t m = cvt_pk_bf16(r0, r1);
          pc[0][i] = h;
          pc[1][i] = m;
          pc[2][i] = cvt_pk_bf16(r0 - __uint_as_float(m << 16), r1 - __uint_as_float(m & 0xFFFF0000u));
        }
#pragma unroll
        for (int p = 0; p < NPX; ++p)
#pragma unroll
          for (int hv = 0; hv < 2; ++hv)
            *reinterpret_cast<uint4 *>(&sm.xs[p][v][16 * c16 + 8 * hv]) =
                make_uint4(pc[p][4 * hv], pc[p][4 * hv + 1], pc[p][4 * hv + 2], pc[p][4 * hv + 3]);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const bf16x2 b2 = __builtin_bit_cast(bf16x2, u[i]);
          ssf = __builtin_amdgcn_fdot2_f32_bf16(b2, b2, ssf, false);
        }
        *reinterpret_cast<uint4 *>(&sm.xs[0][v][16 * c16]) = xc[0];
        *reinterpret_cast<uint4 *>(&sm.xs[0][v][16 * c16 + 8]) = xc[1];
      }
      ssf = group_sum<3>(ssf, lane);
      float nu;
      bool nonfinite = false;
      if (__builtin_expect(!isfinite(ssf), 0)) {
        // rare: an element is not finite, or a float32 square overflowed
        double sd = 0.0;
        bool bad = false;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float xi = F32 ? __uint_as_float(u[i])
                               : __uint_as_float((i & 1) ? (u[i >> 1] & 0xFFFF0000u) : (u[i >> 1] << 16));
          bad |= !isfinite(xi);
          sd = fma(double(xi), double(xi), sd);
        }
#pragma unroll
        for (int o = 4; o > 0; o >>= 1) {
          sd += __shfl_xor(sd, o, kWave);
          bad |= __shfl_xor(static_cast<int>(bad), o, kWave) != 0;
        }
        nonfinite = bad;
        nu = static_cast<float>(sqrt(sd));
      } else {
        nu = __builtin_amdgcn_sqrtf(ssf);
      }
      // the eight lanes of row v write one entry of its vth row each (lane c16,
      // entry c16): ||x|| t_k, or infinity past the K boundaries and for a zero
      // vector, at 0..3; ||x||~ c_k, or 0 past the K + 1 centroids, at 4..7
      bool over = false;
      const uint32_t nb = f16_bits_f32(nu, &over);
      const float n16 = f16_val(nb);
      sm.vth[v][c16] = c16 < 4 ? (c16 < K && nu > 0.0f ? nu * vcoef : INFINITY) : n16 * vcoef;
      if (c16 == 0) {
        sm.nub[v] = nb;
        const Row rw = row_at<GATHER>(a, cur, v, ftpb, fh);
        if (rw.valid) {
          if (nonfinite) flags |= TQ_FLAG_NONFINITE_INPUT;
          if (over) flags |= TQ_FLAG_SCALE_OVERFLOW;
          if (tt.dbg) tt.dbg[size_t(rw.i) * 2] = nu;
        }
      }
    }
    __syncthreads();

    // ---------------------------------------------------------------- B --
    // Row block by row block: the compares of block 0 need only its own
    // products, so they can issue while block 1's products run on the matrix pipe.
    {
      PlaneBits pb[BQ];
      float rr[2] = {0.0f, 0.0f};
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        f32x4 acc[2] = {f32x4{0.0f, 0.0f, 0.0f, 0.0f}, f32x4{0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
          bf16x8 xb[2][NPX];
#pragma unroll
          for (int g2 = 0; g2 < 2; ++g2)
#pragma unroll
            for (int px = 0; px < NPX; ++px)
              xb[g2][px] = *reinterpret_cast<const bf16x8 *>(&sm.xs[px][16 * g2 + li][32 * kc + 8 * lg]);
          const bf16x8 plo = F32 ? pia[NPI - 1][rb][kc]
                                 : *reinterpret_cast<const bf16x8 *>(&sm.plo[F32 ? 0 : cw + 16 * rb + li][32 * kc + 8 * lg]);
#pragma unroll
          for (int px = 0; px < NPX; ++px)
#pragma unroll
            for (int pp = 0; pp < (F32 ? 3 - px : 3); ++pp)
#pragma unroll
              for (int g2 = 0; g2 < 2; ++g2)
                acc[g2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pp < 2 ? pia[pp][rb][kc] : plo, xb[g2][px], acc[g2],
                                                                  0, 0, 0);
        }
        // acc[g2] lane (li, lg) register r: coordinate cw + 16 rb + 4 lg + r of vector 16 g2 + li
#pragma unroll
        for (int g2 = 0; g2 < 2; ++g2) {
          const int vv = 16 * g2 + li;
          const f32x4 th = *reinterpret_cast<const f32x4 *>(&sm.vth[vv][0]);
          const f32x4 cs = *reinterpret_cast<const f32x4 *>(&sm.vth[vv][4]);
          float rho[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float z = acc[g2][r];
            const float az = fabsf(z);
            const bool pos = z >= 0.0f;
            float val = cs[0];
            uint64_t cm[K > 0 ? K : 1];
#pragma unroll
            for (int k = 0; k < K; ++k) {
              const bool c = az >= th[k];
              val = c ? cs[k + 1] : val;
              cm[k] = __ballot(c);
            }
            rho[r] = z - (pos ? val : -val);
            rr[g2] = fmaf(rho[r], rho[r], rr[g2]);
            const uint64_t pm = __ballot(pos);
            // cell = L/2 + m above zero, L/2 - 1 - m below, with m the number of
            // positive boundaries <= |u|; bit q < BQ-1 of m is the parity of the
            // compares at multiples of 2^q (the compares form a thermometer code).
#pragma unroll
            for (int q = 0; q < BQ; ++q) {
              uint64_t bits = pm;
              if (q < BQ - 1) {
                uint64_t mq = 0;
#pragma unroll
                for (int k = 1; k <= K; ++k)
                  if ((k & ((1 << q) - 1)) == 0) mq ^= cm[k - 1];
                bits = ~(mq ^ pm);
              }
              pb[q].put(bits, rb, g2, r);
            }
          }
          // residual pieces for the sketch (written whether or not it runs: no branch
          // here, so the two row blocks stay one straight run of code)
          const uint32_t h01 = cvt_pk_bf16(rho[0], rho[1]), h23 = cvt_pk_bf16(rho[2], rho[3]);
          const uint32_t m01 =
              cvt_pk_bf16(rho[0] - __uint_as_float(h01 << 16), rho[1] - __uint_as_float(h01 & 0xFFFF0000u));
          const uint32_t m23 =
              cvt_pk_bf16(rho[2] - __uint_as_float(h23 << 16), rho[3] - __uint_as_float(h23 & 0xFFFF0000u));
          const int c = cw + 16 * rb + 4 * lg;
          *reinterpret_cast<uint2 *>(&sm.rh[vv][c]) = make_uint2(h01, h23);
          *reinterpret_cast<uint2 *>(&sm.rm[vv][c]) = make_uint2(m01, m23);
        }
      }
#pragma unroll
      for (int g2 = 0; g2 < 2; ++g2) {
        float v = rr[g2];
        v += __shfl_xor(v, 16, kWave);
        v += __shfl_xor(v, 32, kWave);
        if (lg == 0) sm.rr[w][16 * g2 + li] = v;
      }
#pragma unroll
      for (int q = 0; q < BQ; ++q) pb[q].store(sm.wst[q], lane, cw);
    }
    __syncthreads();

    // ---------------------------------------------------------------- D --
    {
      uint32_t rbits = 0;
      if (sk) {
        f32x4 acc[2][2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int g2 = 0; g2 < 2; ++g2) acc[rb][g2] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
          bf16x8 bh[2], bm[2];
#pragma unroll
          for (int g2 = 0; g2 < 2; ++g2) {
            bh[g2] = *reinterpret_cast<const bf16x8 *>(&sm.rh[16 * g2 + li][32 * kc + 8 * lg]);
            bm[g2] = *reinterpret_cast<const bf16x8 *>(&sm.rm[16 * g2 + li][32 * kc + 8 * lg]);
          }
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int g2 = 0; g2 < 2; ++g2)
              acc[rb][g2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sta[0][rb][kc], bh[g2], acc[rb][g2], 0, 0, 0);
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int g2 = 0; g2 < 2; ++g2)
              acc[rb][g2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sta[1][rb][kc], bh[g2], acc[rb][g2], 0, 0, 0);
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int g2 = 0; g2 < 2; ++g2)
              acc[rb][g2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sta[0][rb][kc], bm[g2], acc[rb][g2], 0, 0, 0);
        }
        PlaneBits ps;
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int g2 = 0; g2 < 2; ++g2)
#pragma unroll
            for (int r = 0; r < 4; ++r) ps.put(__ballot(acc[rb][g2][r] >= 0.0f), rb, g2, r);
        ps.store(sm.wst[BQ], lane, cw);
        if (t < QT) {
          float rr = 0.0f;
#pragma unroll
          for (int ww = 0; ww < QW; ++ww) rr += sm.rr[ww][t];
          const float rho = __builtin_amdgcn_sqrtf(rr);
          bool over = false;
          rbits = f16_bits_f32(rho, &over);
          const Row rw = row_at<GATHER>(a, cur, t, ftpb, fh);
          if (rw.valid) {
            if (over) flags |= TQ_FLAG_SCALE_OVERFLOW;
            if (tt.dbg) tt.dbg[size_t(rw.i) * 2 + 1] = rho;
          }
        }
      } else if (t < QT) {
        const Row rw = row_at<GATHER>(a, cur, t, ftpb, fh);
        if (rw.valid && tt.dbg) tt.dbg[size_t(rw.i) * 2 + 1] = 0.0f;
      }
      if (t < QT) sm.scl[t] = sm.nub[t] | (rbits << 16);
      if (GATHER && t < QT) {
        // each row's destination for phase E (read there after the barrier below;
        // rewritten only in the next tile's phase D)
        const Row rw = row_at<GATHER>(a, cur, t, ftpb, fh);
        const bool ok = rw.valid && rw.slot >= 0 && rw.slot < tt.cap;
        if (rw.valid && !ok) flags |= TQ_FLAG_OUT_OF_RANGE;
        sm.gslot[t] = ok ? rw.slot : -1;
        sm.ghead[t] = rw.h;
      }
    }
    __syncthreads();

    // ---------------------------------------------------------------- E --
    if constexpr (GATHER) {
      // rows go to their own slots: scales and token-major records per row; in the
      // value layout one bit per (row, plane, coordinate) word, set or cleared by
      // one atomic (other rows of the same 32-slot block may be written at once)
      const int npl = BQ + (sk ? 1 : 0);
      if (t < QT && sm.gslot[t] >= 0)
        *reinterpret_cast<uint32_t *>(tt.scl + (int64_t(sm.ghead[t]) * tt.cap + sm.gslot[t]) * 2) = sm.scl[t];
      if (tt.layout == TQ_LAYOUT_BLOCK32) {
        for (int c = t; c < npl * QD; c += QN) {
          const int pl = c / QD, cc = c % QD;
          const uint32_t word = *reinterpret_cast<const uint32_t *>(&sm.wst[pl][cc][0]);
          for (int r = 0; r < QT; ++r) {
            const int64_t sl = sm.gslot[r];
            if (sl < 0) continue;
            const int64_t b0 = int64_t(sm.ghead[r]) * (tt.cap / 32) + (sl >> 5);
            uint32_t *dw = pl < BQ ? tt.idx + (b0 * BQ + pl) * QD + cc : tt.sgn + b0 * QD + cc;
            const uint32_t bit = 1u << (sl & 31);
            if ((word >> r) & 1u) atomicOr(dw, bit);
            else atomicAnd(dw, ~bit);
          }
        }
      } else {
        for (int b2 = 0; b2 < npl * 4; b2 += 2 * QW) {
          const int blk = b2 + 2 * w + (lane >> 5), row = lane & 31;
          const int pl = blk >> 2, wd = blk & 3;
          const bool act = blk < npl * 4;
          uint32_t word = act ? *reinterpret_cast<const uint32_t *>(&sm.wst[pl][32 * wd + row][0]) : 0u;
          word = transpose32(word, row);  // lane row now holds row `row`'s word
          const int64_t sl = sm.gslot[row];
          if (act && sl >= 0) {
            const int64_t hs = int64_t(sm.ghead[row]) * tt.cap + sl;
            uint32_t *dw = pl < BQ ? tt.idx + (hs * BQ + pl) * 4 + wd : tt.sgn + hs * 4 + wd;
            *dw = word;
          }
        }
      }
    } else {
      const bool in_range = cur.base >= 0 && cur.base < tt.cap;  // base and cap are multiples of 32
      const int lo = cur.t0 < 0 ? -cur.t0 : 0;
      const int hi = a.n_new - cur.t0 < QT ? a.n_new - cur.t0 : QT;
      const uint32_t vm = hi - lo >= 32 ? 0xFFFFFFFFu : (((1u << (hi - lo)) - 1u) << lo);
      const int npl = BQ + (sk ? 1 : 0);
      if (!in_range) {
        flags |= TQ_FLAG_OUT_OF_RANGE;
      } else {
        const int64_t hs0 = int64_t(cur.h) * tt.cap + cur.base;
        if (t < QT && ((vm >> t) & 1)) *reinterpret_cast<uint32_t *>(tt.scl + (hs0 + t) * 2) = sm.scl[t];
        if (tt.layout == TQ_LAYOUT_BLOCK32) {
          // the (plane, coordinate) words are the value layout's words of this block
          const int64_t b0 = int64_t(cur.h) * (tt.cap / 32) + (cur.base >> 5);
          for (int c = t; c < npl * QD; c += QN) {
            const int pl = c / QD, cc = c % QD;
            const uint32_t word = *reinterpret_cast<const uint32_t *>(&sm.wst[pl][cc][0]);
            uint32_t *dw = pl < BQ ? tt.idx + (b0 * BQ + pl) * QD + cc : tt.sgn + b0 * QD + cc;
            if (vm == 0xFFFFFFFFu) {
              *dw = word;
            } else {
              atomicAnd(dw, ~vm);
              atomicOr(dw, word & vm);
            }
          }
        } else {
          // token-major: transpose each 32 x 32 block (plane, coordinate word) to per-slot words
          for (int b2 = 0; b2 < npl * 4; b2 += 2 * QW) {
            const int blk = b2 + 2 * w + (lane >> 5), row = lane & 31;
            const int pl = blk >> 2, wd = blk & 3;
            const bool act = blk < npl * 4;
            uint32_t word = act ? *reinterpret_cast<const uint32_t *>(&sm.wst[pl][32 * wd + row][0]) : 0u;
            word = transpose32(word, row);  // lane row now holds slot base + row
            if (act && ((vm >> row) & 1)) {
              uint32_t *dw = pl < BQ ? tt.idx + ((hs0 + row) * BQ + pl) * 4 + wd : tt.sgn + (hs0 + row) * 4 + wd;
              *dw = word;
            }
          }
        }
      }
    }
  }
  if (a.status) {
    const uint64_t f1 = __ballot(flags & 1u), f2 = __ballot(flags & 2u), f4 = __ballot(flags & 4u);
    const uint32_t f = (f1 ? 1u : 0u) | (f2 ? 2u : 0u) | (f4 ? 4u : 0u);
    if (lane == 0 && f) atomicOr(a.status, f);
  }
}

// Appends of at most kGatherMaxNew tokens per sequence run on gather tiles when
// they fill at least kGatherMinTiles tiles per tensor.  Fewer vectors go faster on
// one tile per (sequence, head), spread over as many work-groups: a gather tile's
// value records cost 32 x 384 bit updates (atomics) in one work-group, and the
// per-CU atomic rate then sets its time (one-off A/B on the box, one token per
// sequence and 8 heads, K and V: 4 sequences 9.9 us per-sequence tiles against
// 20.8 us gather; 64 sequences 25.7 against 21.4; 512 sequences 138 against 22).
constexpr int kGatherMaxNew = 4;
constexpr int kGatherMinTiles = 8;

template <int BQ, bool F32>
int launch_q(const QuantArgs &a, hipStream_t s) {
  const int64_t nvec = int64_t(a.batch) * a.H * a.n_new;  // vectors per tensor
  const bool gather = a.n_new <= kGatherMaxNew && nvec >= int64_t(kGatherMinTiles) * QT && nvec < (int64_t(1) << 31);
  const int64_t tpb = (int64_t(a.n_new) + QT - 1) / QT + 1;
  const int64_t n1 = gather ? (int64_t(a.batch) * a.H * a.n_new + QT - 1) / QT  // tiles per tensor
                            : int64_t(a.batch) * a.H * tpb;
  const int64_t n_tiles = n1 * (a.n_tensor == 2 ? 2 : 1);
  if (n_tiles >= (int64_t(1) << 31)) return 1;
  // Persistent grid of two work-groups per CU, the occupancy the kernel's
  // registers and LDS are sized for; a grid larger than what fits only queues
  // (work-groups never wait on each other), so no per-process occupancy query or
  // cache is needed.
  constexpr int per_cu = 2;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 256;
  const int64_t full = int64_t(per_cu) * cus;
  const unsigned grid = static_cast<unsigned>(n_tiles < full ? n_tiles : full);
  if (grid == 0) return 0;
  if (gather)
    hipLaunchKernelGGL((quantize_mfma<BQ, F32, true>), dim3(grid), dim3(QN), 0, s, a, static_cast<uint32_t>(n_tiles),
                       static_cast<uint32_t>(n1), make_fastdiv(static_cast<uint32_t>(a.n_new)),
                       make_fastdiv(static_cast<uint32_t>(a.H)));
  else
    hipLaunchKernelGGL((quantize_mfma<BQ, F32, false>), dim3(grid), dim3(QN), 0, s, a, static_cast<uint32_t>(n_tiles),
                       static_cast<uint32_t>(n1), make_fastdiv(static_cast<uint32_t>(tpb)),
                       make_fastdiv(static_cast<uint32_t>(a.H)));
  return hipGetLastError() != hipSuccess;
}

// ===========================================================================
// d = m = 256.  The bf16 pieces of Pi and S~ (512 or 640 KB) exceed what a CU
// holds in registers and LDS together, so they stream from L2 (every CU reads
// the same matrices, which stay resident there) into registers: a 32-column
// slice of the wave's rows at a time, WPD slices ahead of the products.  The
// tile grows to 128 vectors (four 32-slot blocks), so each matrix element
// fetched serves 128 products, and the input tile and then the residual's two
// pieces share one LDS region.  Work-group: 8 waves, one per CU; wave w owns
// coordinates and sketch rows 32w .. 32w+31.  bf16 input only (exact in one
// piece); Pi takes its hi and mid pieces, and lo too at b' = 3, where the
// residual is smallest relative to ||x|| and ||r||'s tolerance needs it.
// Phases per tile as above: A (input to LDS, norms), B (z = Pi x, cells,
// residual), D (sketch), E (records); the next tile's input is loaded into
// registers after the sketch's products, so that the in-order completion of
// loads never makes a matrix slice wait for HBM.
// ===========================================================================
constexpr int WD = 256;      // d = m
constexpr int WT = 128;      // vectors per tile
constexpr int WW = 8;        // waves per work-group
constexpr int WN = 64 * WW;  // threads per work-group
constexpr int WPD = 2;       // matrix slices in flight ahead of the products
constexpr int WPF = 2;       // column operand reads in flight ahead of the products

template <int BQ>
struct WSmem {
  union {
    __align__(16) uint16_t xs[WT * WD];     // input (bf16 bits), swizzled rows
    __align__(16) uint16_t rp[2][WT * WD];  // residual: hi and mid pieces, swizzled rows
  } u;
  __align__(16) float vth[WT][8];                // per vector: ||x|| t_k at 0..2, ||x||~ c_k at 4..7
  __align__(16) float rr[WW][WT];                // ||rho||^2 over each wave's coordinates
  __align__(16) uint16_t wst[BQ + 1][4][WD][2];  // words (plane, block, coordinate); plane BQ: signs
  __align__(16) uint32_t nub[WT];                // fp16 bits of ||x||
  __align__(16) uint32_t scl[WT];                // nu bits | rho bits << 16
};

// Element index of 16-byte chunk `chunk` (0..31) of row `row` in an operand
// tile: rows are unpadded and the chunk index is XORed with the row's low four
// bits.  An MFMA operand read (16 rows, four consecutive chunks) then spreads
// over all LDS banks; a padded row stride of 16 bytes costs about four stall
// cycles per 128-bit read on gfx950 (measured with the bank-conflict counter).
__device__ inline int swz(int row, int chunk) { return row * WD + 8 * (chunk ^ (row & 15)); }

// The MFMA column operand of step (kc, cb): row 16 cb + li, chunk 4 kc + lg.
// With li = 4 lh + ll the chunk is 4 (kc ^ lh) + (lg ^ ll), so the element
// index is base[kc & 3] + WD * 16 cb + 32 (kc & 4): four per-lane bases, and
// everything else an immediate offset of the LDS read.
struct OpBase {
  int b[4];
  __device__ inline OpBase(int li, int lg) {
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = li * WD + 32 * (j ^ (li >> 2)) + 8 * (lg ^ (li & 3));
  }
  __device__ inline int at(int kc, int cb) const { return b[kc & 3] + WD * 16 * cb + 32 * (kc & 4); }
};

// PlaneBits over the four 32-slot blocks of a tile: pk[blk] gathers the masks
// of column blocks 2 blk and 2 blk + 1 in the lane order PlaneBits uses.
struct PlaneBits4 {
  uint32_t pk[4] = {0u, 0u, 0u, 0u};
  __device__ inline void put(uint64_t m, int rb, int cb, int r) {
    const int l = rb * 16 + r * 4 + (cb & 1) * 2;
    pk[cb >> 1] = wlane(static_cast<uint32_t>(m), l, pk[cb >> 1]);
    pk[cb >> 1] = wlane(static_cast<uint32_t>(m >> 32), l + 1, pk[cb >> 1]);
  }
  __device__ inline void store(uint16_t (*w)[WD][2], int lane, int c0) const {
    if (lane < 32) {
      const int rb = lane >> 4, r = (lane >> 2) & 3, g2 = (lane >> 1) & 1, hh = lane & 1;
      const int c = c0 + 16 * rb + 8 * hh + r;
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        w[blk][c][g2] = static_cast<uint16_t>(pk[blk]);
        w[blk][c + 4][g2] = static_cast<uint16_t>(pk[blk] >> 16);
      }
    }
  }
};

// Row v of a 128-vector tile, 16-byte chunks 4 i + q4 (i = 0..7): four lanes
// read 64 contiguous bytes of a row per instruction.  Zeros outside the tokens.
// The input is read once: non-temporal loads, so that it streams through L2
// without evicting the matrix slices every CU reads there.
__device__ inline void load_rows_w(const QuantArgs &a, const Tile &T, int v, int q4, uint4 *r) {
  const int tok = T.t0 + v;
  if (tok >= 0 && tok < a.n_new) {
    const size_t row = (size_t(T.b) * a.H + T.h) * size_t(a.n_new) + tok;
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 *p = reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(a.t.x) + row * WD) + q4;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const u32x4 v = __builtin_nontemporal_load(p + 4 * i);
      r[i] = make_uint4(v.x, v.y, v.z, v.w);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = make_uint4(0, 0, 0, 0);
  }
}

// One 32-column slice (columns 32 kc + 8 lg .. + 7) of the wave's two row
// blocks of NP pieces of a 256 x 256 matrix split as [3][256][256], through a
// buffer resource: the lane's byte offset voff in a VGPR, the slice's in an SGPR.
template <int NP>
__device__ inline void load_slice(__amdgpu_buffer_rsrc_t m, int voff, int kc, bf16x8 (*dst)[2]) {
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
      dst[p][rb] = __builtin_bit_cast(
          bf16x8, __builtin_amdgcn_raw_buffer_load_b128(m, voff, 2 * ((p * WD + 16 * rb) * WD + 32 * kc), 0));
}

template <int BQ, int NPI>
__global__ __launch_bounds__(WN, 1) void quantize_wide(QuantArgs a, uint32_t n_tiles, uint32_t n1, FastDiv ftpb, FastDiv fh) {
  constexpr int L = 1 << BQ;
  constexpr int K = L / 2 - 1;  // positive boundaries
  __shared__ WSmem<BQ> sm;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, li = lane & 15, lg = lane >> 4;
  const int v = t >> 2, q4 = t & 3;  // phase A: row v, chunks 4 i + q4
  const int cw = 32 * w;             // first coordinate / sketch row of this wave
  const bool sk = a.t.sketch != 0;
  // lane (li, lg) of a slice: rows cw + 16 rb + li, columns 32 kc + 8 lg .. + 7
  const __amdgpu_buffer_rsrc_t prot =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(a.rot_hml), 0, 3 * WD * WD * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t pst =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(a.st_hml), 0, 3 * WD * WD * 2, 0x00020000);
  const int moff = 2 * ((cw + li) * WD + 8 * lg);
  const OpBase ob(li, lg);

  float tpos[K > 0 ? K : 1], cpos[K + 1];
#pragma unroll
  for (int k = 0; k < K; ++k) tpos[k] = a.t.cb.thr[L / 2 + k];
#pragma unroll
  for (int k = 0; k <= K; ++k) cpos[k] = a.t.cb.cen[L / 2 + k];

  uint32_t flags = 0;
  uint4 xr[8];
  uint32_t tile = blockIdx.x;
  Tile T{};
  if (tile < n_tiles) {
    T = tile_at<WT>(a, tile, n1, ftpb, fh);
    load_rows_w(a, T, v, q4, xr);
  }
  for (; tile < n_tiles; tile += gridDim.x) {
    const Tile cur = T;
    const QuantTensorArgs &tt = a.t;  // one tensor per launch at d = 256
    const uint32_t nxt = tile + gridDim.x;
    if (cur.t0 >= a.n_new) {  // no token falls in this tile (uniform)
      if (nxt < n_tiles) {
        T = tile_at<WT>(a, nxt, n1, ftpb, fh);
        load_rows_w(a, T, v, q4, xr);
      }
      continue;
    }
    bf16x8 pa[WPD + 1][NPI][2];  // ring of slices of Pi
#pragma unroll
    for (int kc = 0; kc < WPD; ++kc) load_slice<NPI>(prot, moff, kc, pa[kc]);

    // ---------------------------------------------------------------- A --
    {
      const uint32_t *u = reinterpret_cast<const uint32_t *>(xr);
      float ssf = 0.0f;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const bf16x2 b2 = __builtin_bit_cast(bf16x2, u[i]);
        ssf = __builtin_amdgcn_fdot2_f32_bf16(b2, b2, ssf, false);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) *reinterpret_cast<uint4 *>(&sm.u.xs[swz(v, 4 * i + q4)]) = xr[i];
      ssf = group_sum<2>(ssf, lane);
      float nu;
      bool nonfinite = false;
      if (__builtin_expect(!isfinite(ssf), 0)) {
        // rare: an element is not finite, or a float32 square overflowed
        double sd = 0.0;
        bool bad = false;
#pragma unroll
        for (int i = 0; i < 64; ++i) {
          const float xi = __uint_as_float((i & 1) ? (u[i >> 1] & 0xFFFF0000u) : (u[i >> 1] << 16));
          bad |= !isfinite(xi);
          sd = fma(double(xi), double(xi), sd);
        }
#pragma unroll
        for (int o = 1; o < 4; o <<= 1) {
          sd += __shfl_xor(sd, o, kWave);
          bad |= __shfl_xor(static_cast<int>(bad), o, kWave) != 0;
        }
        nonfinite = bad;
        nu = static_cast<float>(sqrt(sd));
      } else {
        nu = __builtin_amdgcn_sqrtf(ssf);
      }
      if (q4 == 0) {
        bool over = false;
        const uint32_t nb = f16_bits_f32(nu, &over);
        const float n16 = f16_val(nb);
        f32x4 th = {INFINITY, INFINITY, INFINITY, INFINITY}, cs = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int k = 0; k < K; ++k) th[k] = nu > 0.0f ? nu * tpos[k] : INFINITY;
#pragma unroll
        for (int k = 0; k <= K; ++k) cs[k] = n16 * cpos[k];
        *reinterpret_cast<f32x4 *>(&sm.vth[v][0]) = th;
        *reinterpret_cast<f32x4 *>(&sm.vth[v][4]) = cs;
        sm.nub[v] = nb;
        const int tok = cur.t0 + v;
        if (tok >= 0 && tok < a.n_new) {
          if (nonfinite) flags |= TQ_FLAG_NONFINITE_INPUT;
          if (over) flags |= TQ_FLAG_SCALE_OVERFLOW;
          if (tt.dbg) tt.dbg[((int64_t(cur.b) * a.H + cur.h) * a.n_new + tok) * 2] = nu;
        }
      }
    }
    __syncthreads();

    // ---------------------------------------------------------------- B --
    f32x4 acc[2][8];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) acc[rb][cb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    // Column operands WPF steps ahead of their products over the 64 (kc, cb)
    // steps; the fences keep the scheduler from hoisting every step's operand
    // (registers).
    bf16x8 xb[WPF + 1];
#pragma unroll
    for (int s0 = 0; s0 < WPF; ++s0)
      xb[s0] = *reinterpret_cast<const bf16x8 *>(&sm.u.xs[ob.at(s0 >> 3, s0 & 7)]);
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) {
      if (kc + WPD < 8) load_slice<NPI>(prot, moff, kc + WPD, pa[(kc + WPD) % (WPD + 1)]);
      const int sl = kc % (WPD + 1);
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) {
        const int st = 8 * kc + cb, sn = st + WPF;
        if (sn < 64)
          xb[sn % (WPF + 1)] = *reinterpret_cast<const bf16x8 *>(&sm.u.xs[ob.at(sn >> 3, sn & 7)]);
#pragma unroll
        for (int p = 0; p < NPI; ++p)
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
            acc[rb][cb] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[sl][p][rb], xb[st % (WPF + 1)], acc[rb][cb], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // acc[rb][cb] lane (li, lg) register r: coordinate cw + 16 rb + 4 lg + r of vector 16 cb + li;
    // it is overwritten with the residual.
    {
      PlaneBits4 pb[BQ];
      float rr[8];
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) {
        const int vv = 16 * cb + li;
        const f32x4 th = *reinterpret_cast<const f32x4 *>(&sm.vth[vv][0]);
        const f32x4 cs = *reinterpret_cast<const f32x4 *>(&sm.vth[vv][4]);
        rr[cb] = 0.0f;
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float z = acc[rb][cb][r];
            const float az = fabsf(z);
            const bool pos = z >= 0.0f;
            float val = cs[0];
            uint64_t cm[K > 0 ? K : 1];
#pragma unroll
            for (int k = 0; k < K; ++k) {
              const bool c = az >= th[k];
              val = c ? cs[k + 1] : val;
              cm[k] = __ballot(c);
            }
            const float rho = z - (pos ? val : -val);
            acc[rb][cb][r] = rho;
            rr[cb] = fmaf(rho, rho, rr[cb]);
            const uint64_t pm = __ballot(pos);
            // cell index bits from the thermometer-coded compares, as for d = 128
#pragma unroll
            for (int q = 0; q < BQ; ++q) {
              uint64_t bits = pm;
              if (q < BQ - 1) {
                uint64_t mq = 0;
#pragma unroll
                for (int k = 1; k <= K; ++k)
                  if ((k & ((1 << q) - 1)) == 0) mq ^= cm[k - 1];
                bits = ~(mq ^ pm);
              }
              pb[q].put(bits, rb, cb, r);
            }
          }
      }
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) {
        float x = rr[cb];
        x += __shfl_xor(x, 16, kWave);
        x += __shfl_xor(x, 32, kWave);
        if (lg == 0) sm.rr[w][16 * cb + li] = x;
      }
#pragma unroll
      for (int q = 0; q < BQ; ++q) pb[q].store(sm.wst[q], lane, cw);
    }
    __syncthreads();  // every wave is done with the input tile
    bf16x8 ps[WPD + 1][2][2];  // ring of slices of S~ (hi, mid)
    if (sk) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) {
          const f32x4 rho = acc[rb][cb];
          const uint32_t h01 = cvt_pk_bf16(rho[0], rho[1]), h23 = cvt_pk_bf16(rho[2], rho[3]);
          const uint32_t m01 =
              cvt_pk_bf16(rho[0] - __uint_as_float(h01 << 16), rho[1] - __uint_as_float(h01 & 0xFFFF0000u));
          const uint32_t m23 =
              cvt_pk_bf16(rho[2] - __uint_as_float(h23 << 16), rho[3] - __uint_as_float(h23 & 0xFFFF0000u));
          // coordinates cw + 16 rb + 4 lg .. + 3: half lg & 1 of chunk 4 w + 2 rb + lg / 2
          const int e = swz(16 * cb + li, 4 * w + 2 * rb + (lg >> 1)) + 4 * (lg & 1);
          *reinterpret_cast<uint2 *>(&sm.u.rp[0][e]) = make_uint2(h01, h23);
          *reinterpret_cast<uint2 *>(&sm.u.rp[1][e]) = make_uint2(m01, m23);
        }
#pragma unroll
      for (int kc = 0; kc < WPD; ++kc) load_slice<2>(pst, moff, kc, ps[kc]);
    }
    if (!sk && nxt < n_tiles) {
      T = tile_at<WT>(a, nxt, n1, ftpb, fh);
      load_rows_w(a, T, v, q4, xr);
    }
    __syncthreads();

    // ---------------------------------------------------------------- D --
    {
      uint32_t rbits = 0;
      if (sk) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int cb = 0; cb < 8; ++cb) acc[rb][cb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        bf16x8 bh[WPF + 1], bm[WPF + 1];
#pragma unroll
        for (int s0 = 0; s0 < WPF; ++s0) {
          bh[s0] = *reinterpret_cast<const bf16x8 *>(&sm.u.rp[0][ob.at(s0 >> 3, s0 & 7)]);
          bm[s0] = *reinterpret_cast<const bf16x8 *>(&sm.u.rp[1][ob.at(s0 >> 3, s0 & 7)]);
        }
#pragma unroll
        for (int kc = 0; kc < 8; ++kc) {
          if (kc + WPD < 8) load_slice<2>(pst, moff, kc + WPD, ps[(kc + WPD) % (WPD + 1)]);
          const int sl = kc % (WPD + 1);
#pragma unroll
          for (int cb = 0; cb < 8; ++cb) {
            const int st = 8 * kc + cb, sn = st + WPF, q = st % (WPF + 1);
            if (sn < 64) {
              const int e = ob.at(sn >> 3, sn & 7);
              bh[sn % (WPF + 1)] = *reinterpret_cast<const bf16x8 *>(&sm.u.rp[0][e]);
              bm[sn % (WPF + 1)] = *reinterpret_cast<const bf16x8 *>(&sm.u.rp[1][e]);
            }
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
              acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ps[sl][0][rb], bh[q], acc[rb][cb], 0, 0, 0);
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
              acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ps[sl][1][rb], bh[q], acc[rb][cb], 0, 0, 0);
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
              acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ps[sl][0][rb], bm[q], acc[rb][cb], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        // the next tile's input: issued after the last matrix slice, since a
        // wait for a slice issued later would also wait for these HBM loads
        if (nxt < n_tiles) {
          T = tile_at<WT>(a, nxt, n1, ftpb, fh);
          load_rows_w(a, T, v, q4, xr);
        }
        PlaneBits4 pbs;
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int cb = 0; cb < 8; ++cb)
#pragma unroll
            for (int r = 0; r < 4; ++r) pbs.put(__ballot(acc[rb][cb][r] >= 0.0f), rb, cb, r);
        pbs.store(sm.wst[BQ], lane, cw);
        if (t < WT) {
          float rr = 0.0f;
#pragma unroll
          for (int ww = 0; ww < WW; ++ww) rr += sm.rr[ww][t];
          const float rho = __builtin_amdgcn_sqrtf(rr);
          bool over = false;
          rbits = f16_bits_f32(rho, &over);
          const int tok = cur.t0 + t;
          if (tok >= 0 && tok < a.n_new) {
            if (over) flags |= TQ_FLAG_SCALE_OVERFLOW;
            if (tt.dbg) tt.dbg[((int64_t(cur.b) * a.H + cur.h) * a.n_new + tok) * 2 + 1] = rho;
          }
        }
      } else if (t < WT) {
        const int tok = cur.t0 + t;
        if (tok >= 0 && tok < a.n_new && tt.dbg)
          tt.dbg[((int64_t(cur.b) * a.H + cur.h) * a.n_new + tok) * 2 + 1] = 0.0f;
      }
      if (t < WT) sm.scl[t] = sm.nub[t] | (rbits << 16);
    }
    __syncthreads();

    // ---------------------------------------------------------------- E --
    {
      // block blk holds slots base + 32 blk ..; its tokens t0 + 32 blk + j, j in [lo, hi)
      uint32_t vm[4];
      bool inr[4];
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        const int tb = cur.t0 + 32 * blk;
        const int lo = tb < 0 ? -tb : 0;
        const int hi = a.n_new - tb < 32 ? a.n_new - tb : 32;
        vm[blk] = hi <= lo ? 0u : hi - lo >= 32 ? 0xFFFFFFFFu : (((1u << (hi - lo)) - 1u) << lo);
        const int64_t sb = cur.base + 32 * blk;  // base and cap are multiples of 32
        inr[blk] = sb >= 0 && sb < tt.cap;
        if (vm[blk] != 0u && !inr[blk]) flags |= TQ_FLAG_OUT_OF_RANGE;
      }
      const int npl = BQ + (sk ? 1 : 0);
      const int64_t hs0 = int64_t(cur.h) * tt.cap + cur.base;
      if (t < WT && ((vm[t >> 5] >> (t & 31)) & 1) && inr[t >> 5])
        *reinterpret_cast<uint32_t *>(tt.scl + (hs0 + t) * 2) = sm.scl[t];
      if (tt.layout == TQ_LAYOUT_BLOCK32) {
        // the (plane, block, coordinate) words are the value layout's words
        const int64_t b0 = int64_t(cur.h) * (tt.cap / 32) + (cur.base >> 5);
        for (int c = t; c < npl * 4 * WD; c += WN) {
          const int pl = c / (4 * WD), blk = (c / WD) & 3, cc = c % WD;
          const uint32_t m = vm[blk];
          if (m == 0u || !inr[blk]) continue;
          const uint32_t word = *reinterpret_cast<const uint32_t *>(&sm.wst[pl][blk][cc][0]);
          uint32_t *dw = pl < BQ ? tt.idx + ((b0 + blk) * BQ + pl) * WD + cc : tt.sgn + (b0 + blk) * WD + cc;
          if (m == 0xFFFFFFFFu) {
            *dw = word;
          } else {
            atomicAnd(dw, ~m);
            atomicOr(dw, word & m);
          }
        }
      } else {
        // token-major: transpose each 32 x 32 block (plane, block, coordinate word) to per-slot words
        for (int b2 = 0; b2 < npl * 32; b2 += 2 * WW) {
          const int bid = b2 + 2 * w + (lane >> 5), row = lane & 31;
          const int pl = bid >> 5, blk = (bid >> 3) & 3, wd = bid & 7;
          uint32_t word = *reinterpret_cast<const uint32_t *>(&sm.wst[pl][blk][32 * wd + row][0]);
          word = transpose32(word, row);  // lane row now holds slot base + 32 blk + row
          if (((vm[blk] >> row) & 1) && inr[blk]) {
            const int64_t slot = hs0 + 32 * blk + row;
            uint32_t *dw = pl < BQ ? tt.idx + (slot * BQ + pl) * (WD / 32) + wd : tt.sgn + slot * (WD / 32) + wd;
            *dw = word;
          }
        }
      }
    }
  }
  if (a.status) {
    const uint64_t f1 = __ballot(flags & 1u), f2 = __ballot(flags & 2u), f4 = __ballot(flags & 4u);
    const uint32_t f = (f1 ? 1u : 0u) | (f2 ? 2u : 0u) | (f4 ? 4u : 0u);
    if (lane == 0 && f) atomicOr(a.status, f);
  }
}

template <int BQ>
int launch_w(const QuantArgs &a, hipStream_t s) {
  if (a.n_tensor != 1) return 1;  // one tensor per launch at d = 256 (its registers are full)
  const int64_t tpb = (int64_t(a.n_new) + 31 + WT - 1) / WT;
  const int64_t n1 = int64_t(a.batch) * a.H * tpb;
  const int64_t n_tiles = n1;
  if (n_tiles >= (int64_t(1) << 31)) return 1;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 256;
  const unsigned grid = static_cast<unsigned>(n_tiles < cus ? n_tiles : cus);
  if (grid == 0) return 0;
  constexpr int NPI = BQ == 3 ? 3 : 2;
  hipLaunchKernelGGL((quantize_wide<BQ, NPI>), dim3(grid), dim3(WN), 0, s, a, static_cast<uint32_t>(n_tiles),
                     static_cast<uint32_t>(n1), make_fastdiv(static_cast<uint32_t>(tpb)), make_fastdiv(static_cast<uint32_t>(a.H)));
  return hipGetLastError() != hipSuccess;
}

}  // namespace

int launch_quantize_fast(int d, const QuantArgs &a, hipStream_t s) {
  const bool f32 = a.dtype == TQ_F32;
  if (d == WD && !f32) {
    switch (a.t.bq) {
      case 1: return launch_w<1>(a, s);
      case 2: return launch_w<2>(a, s);
      case 3: return launch_w<3>(a, s);
      default: return 1;
    }
  }
  if (d != QD) return 1;
  switch (a.t.bq) {
    case 1: return f32 ? launch_q<1, true>(a, s) : launch_q<1, false>(a, s);
    case 2: return f32 ? launch_q<2, true>(a, s) : launch_q<2, false>(a, s);
    case 3: return f32 ? launch_q<3, true>(a, s) : launch_q<3, false>(a, s);
    default: return 1;
  }
}

}  // namespace tq
