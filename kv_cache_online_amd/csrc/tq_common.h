// Internal declarations shared by the libtq translation units (not part of the ABI).
#pragma once

#include <cstddef>
#include <cstdint>

#include "tq.h"

namespace tq {

// ---------------------------------------------------------------- prep blob --
// Device-side matrices derived on the host from Pi and S (d == m):
//   rotT   fp32 [d][d]   rotT[k][j] = Pi[j][k]
//   stT    fp32 [d][m]   stT[j][i]  = S~[i][j],  S~ = S Pi^T (float64, then fp32)
//   projT  fp32 [d][m]   projT[k][i] = S[i][k]
//   rot_hml bf16 [3][d][d]  Pi split hi/mid/lo (hi + mid + lo == fp32 Pi exactly)
//   st_hml  bf16 [3][m][d]  S~ split hi/mid/lo
//   stnorm fp32 [m]      row norms ||S~_i||_2
// Every section starts on a 256-byte boundary after a 256-byte header.
struct PrepLayout {
  size_t rotT, stT, projT, rot_hml, st_hml, stnorm, total;
};

constexpr uint32_t kPrepMagic = 0x31505154u;  // "TQP1"

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline PrepLayout prep_layout(int d, int m) {
  PrepLayout L{};
  size_t o = 256;
  L.rotT = o;    o = align256(o + size_t(d) * d * 4);
  L.stT = o;     o = align256(o + size_t(d) * m * 4);
  L.projT = o;   o = align256(o + size_t(d) * m * 4);
  L.rot_hml = o; o = align256(o + size_t(3) * d * d * 2);
  L.st_hml = o;  o = align256(o + size_t(3) * m * d * 2);
  L.stnorm = o;  o = align256(o + size_t(m) * 4);
  L.total = o;
  return L;
}

// ------------------------------------------------------ query operand shape --
// The decode's score products (v_mfma_scale_f32_16x16x128_f8f6f4) take the
// queries as fp6 (e2m3) base-16 digits, kQDigits per entry, and the key bit
// planes as fp4 (e2m1).  A product's 16 rows are (query head, digit slot) for a
// group of G heads: q_slots(G) = 16 / G slots per head, q_products(G) products
// per plane and 128-coordinate chunk to hold every digit.
constexpr int kQDigits = 6;
constexpr int q_slots(int G) { return 16 / G; }
constexpr int q_products(int G) { return (kQDigits + 16 / G - 1) / (16 / G); }
// Bytes of one group's operands: 5 plane slots x d / 128 chunks x products x 64
// lanes x 32 bytes (six used), and 64 lanes x 32 scale bytes.
constexpr size_t q_operand_bytes(int d, int G) { return size_t(5) * (d / 128) * q_products(G) * 64 * 32; }
constexpr size_t q_scale_bytes() { return size_t(64) * 32; }

// --------------------------------------------------------------- decode plan --
// Token splits of the decode partial pass.  The same plan sizes the workspace
// and the launch, so both derive it from (batch, kv heads, max_len) alone.
struct DecodePlan {
  int32_t split_tokens;  // tokens per split, a multiple of 256
  int32_t n_split;       // splits per (sequence, kv head), covering max_len + 63 slots
  int32_t fast;          // 1: matrix-core kernels; 0: reference-grade kernels
  int32_t rb;            // row blocks of 16 (= G / 4) in the matrix-core kernels
  size_t off_qr, off_qs, off_part, off_qop, off_qscale, off_smax, total;  // workspace byte offsets
  int32_t part_stride;   // floats per partial record: 4 + d + m (matrix-core layout; the reference kernels use 2 + d + m)
};

DecodePlan decode_plan(const tq_config &cfg, int32_t batch, int32_t max_len);

// ----------------------------------------------------- kernel-side arguments --
struct CodebookF32 {
  float thr[TQ_MAX_LEVELS - 1];
  float cen[TQ_MAX_LEVELS];
  int32_t levels;
};

struct QuantTensorArgs {
  const void *x;         // [batch][H][n_new][d]
  uint32_t *idx;
  uint32_t *sgn;
  uint16_t *scl;
  int64_t cap;
  int32_t layout;
  int32_t bq;            // b'
  int32_t sketch;
  CodebookF32 cb;
  float *dbg;            // [batch][H][n_new][2] or null
};

struct QuantArgs {
  // t, and t2 when n_tensor == 2: tensors with the same spec (b', sketch,
  // codebook) quantized by one launch, whose tiles run over t's then t2's
  QuantTensorArgs t, t2;
  int32_t n_tensor;
  int32_t dtype;         // tq_dtype
  int32_t batch, H, n_new;
  const int64_t *dst;
  const float *rotT;
  const float *stT;
  const uint16_t *rot_hml;  // Pi as three bf16 pieces [3][d][d]
  const uint16_t *st_hml;   // S~ as three bf16 pieces [3][m][d]
  uint32_t *status;
};

struct DecodeTensorArgs {
  const uint32_t *idx;
  const uint32_t *sgn;
  const uint16_t *scl;
  int64_t cap;
  int32_t bq;
  int32_t sketch;
  CodebookF32 cb;
};

struct DecodeArgs {
  DecodeTensorArgs k, v;
  double walsh_k[4];     // key codebook Walsh coefficients, planes ordered s0, s1, s2, s0 s1 s2
  double walsh_v[4];     // value codebook, same order
  // query operands of the matrix-core scores, per (sequence, kv head) group of G
  // query heads: qop [group][plane slot 5][d / 128][q_products(G)][lane 64][8
  // words] fp6 digits (six words used), qscale [group][lane 64][32] their E8M0
  // scale bytes, byte (plane * d / 128 + chunk) * q_products(G) + product
  uint32_t *qop;
  uint8_t *qscale;
  const void *q;         // [batch][Hq][d]
  int32_t dtype;
  int32_t batch, Hkv, Hq, G;
  const int64_t *seq_start;
  const int32_t *seq_len;
  int32_t max_len;       // host bound on seq_len: longer sequences are clipped and flagged
  float sm_scale;
  float kappa;           // sqrt(pi/2) / m
  const float *rot;      // Pi [d][d]
  const float *proj;     // S [m][d]
  const float *rotT;
  const float *projT;
  const float *stnorm;   // row norms of S~ = S Pi^T [m]
  float *qr;             // [batch][Hq][d]
  float *qs;             // [batch][Hq][m]
  float *part;           // [batch][Hq][n_split][2 + d + m]
  int32_t split_tokens, n_split;
  float *out;            // [batch][Hq][d]
  uint32_t *status;
  double qbase;          // scale of the scores: sm_scale log2(e) (decode, base-2 scores), 1 (raw scores)
  // key scoring (tq_score_keys): every block reads key head kv_fixed (-1: its own),
  // slots [fix_start, fix_start + fix_len) when seq_start is null, and writes raw
  // scores [Hq][score_ld] instead of attention partials
  int32_t kv_fixed;
  int64_t fix_start;
  int32_t fix_len;
  float *scores;
  int64_t score_ld;
  float *score_dummy;  // 64 words that scoring lanes outside the range write instead
  // Sparse V decode: a position's value is kept when its score (base 2) reaches the
  // head's largest score plus sparse_thr = log2(tau); smax [batch][Hq][n_split]
  // holds every split's largest score per head
  float sparse_thr;
  float *smax;
};

// Host launchers (defined in the .hip translation units).  Return hipError_t.
int launch_quantize(int d, const QuantArgs &a, hipStream_t s);
int launch_quantize_fast(int d, const QuantArgs &a, hipStream_t s);
int launch_decode(int d, const DecodeArgs &a, hipStream_t s);
int launch_decode_fast(int d, int rb, const DecodeArgs &a, hipStream_t s, bool sparse);
int launch_score_fast(int d, const DecodeArgs &a, hipStream_t s);

}  // namespace tq
