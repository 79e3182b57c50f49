/*
 * tq.h -- C ABI of libtq: online compression of LLM key/value vectors into a
 * bit-packed cache, and decode attention that reads that cache, on MI355X
 * (gfx950).
 *
 * The method (sources cited by page title and section):
 *   [softpro 1.2]  ast-softpro.ru, "Технология TurboQuant и её применение с
 *                  локальными LLM", section 1.2 "Как работает TurboQuant".
 *                  Stage 1: every KV vector is multiplied by a random
 *                  orthogonal matrix and each rotated coordinate is quantized
 *                  independently by an MSE-optimal Lloyd-Max quantizer with
 *                  b-1 bits.  Stage 2 (QJL): the residual
 *                  r = x - DEQUANT_mse(Q_mse(x)) is projected by a random
 *                  Gaussian matrix S, only sign(S r) is kept, and ||r||_2 is
 *                  kept for reconstruction.
 *   [kiosk method] kiosknews.app, "3 бита вместо 16: разбираем TurboQuant и
 *                  когда его реально стоит включать", section "Как работает
 *                  TurboQuant": the codebook is computed once for the known
 *                  post-rotation distribution, stored, and needs no
 *                  calibration.
 *   [kiosk python] same page, section "Python + HuggingFace": quantize
 *                  returns (indices, norms) -- a per-vector norm is stored.
 *
 * Readings taken where the pages are silent:
 *   - the quantizer acts on u = Pi x / ||x||; the codebook is the Lloyd-Max
 *     quantizer of N(0, sigma^2), sigma = 1/sqrt(d);
 *   - ||x|| and ||r|| are stored as IEEE fp16 (round to nearest even from the
 *     exact value; > 65504 saturates and raises TQ_FLAG_SCALE_OVERFLOW);
 *   - the cell decision uses the unrounded ||x||; the residual uses the
 *     stored fp16 norm: r = x - Pi^T (nu16 * c[idx]);
 *   - a cell index is the number of thresholds t_k with u >= t_k;
 *   - S is m x d with N(0,1) entries, m == d; a sign bit is 1 when (S r)_i >= 0;
 *   - the residual is reconstructed as sqrt(pi/2)/m * rho16 * S^T (2 sgn - 1)
 *     (the scaling that makes <q, r_hat> unbiased over S);
 *   - decode attention is softmax(q . k_hat / sqrt(d)) . v_hat over all cached
 *     tokens of the sequence, query head h reading kv head h / G.
 *
 * Conventions for every call:
 *   - Ownership: the caller allocates and frees every buffer.  libtq
 *     allocates nothing, never synchronizes and keeps no state between calls.
 *     Host structs are only read during the call.
 *   - Device calls enqueue work on `stream` and return at once.  Argument
 *     errors are returned synchronously as negative tq_status values and
 *     nothing is enqueued.  A launch failure returns TQ_ERR_LAUNCH.
 *     Data-dependent conditions never fail a call: they set bits in the
 *     caller's device status word (OR-ed, never cleared by libtq).
 *   - Device pointers must be 16-byte aligned unless the call says otherwise
 *     (status words, sequence lengths and search scores: 4 bytes; sequence
 *     starts and destination slots: 8 bytes).
 *   - Reentrant: concurrent calls on different streams with disjoint outputs
 *     are safe.
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TQ_OK = 0,
  TQ_ERR_INVALID_ARG = -1,   /* null pointer, bad size, misaligned pointer   */
  TQ_ERR_UNSUPPORTED = -2,   /* valid but not implemented (e.g. d not 64/128/256) */
  TQ_ERR_WORKSPACE = -3,     /* workspace smaller than tq_decode_workspace_bytes */
  TQ_ERR_LAUNCH = -4,        /* kernel launch failed (hipGetLastError)       */
  TQ_ERR_NO_CONVERGENCE = -5 /* Lloyd-Max did not converge                   */
} tq_status;

/* TQ_DTYPE_RANGE_ widens the enum's range to all of int32, so that reading any
 * value a caller passes (and rejecting it with TQ_ERR_INVALID_ARG) is defined. */
typedef enum { TQ_F32 = 0, TQ_BF16 = 1, TQ_DTYPE_RANGE_ = -2147483647 - 1 } tq_dtype;

/* Cache layouts (bit k of a uint32 word is its k-th least significant bit;
 * index plane q holds bit q of the cell index; a sign bit is 1 for (S r)_i >= 0):
 *   TQ_LAYOUT_TOKEN_MAJOR: idx[head][slot][q][d/32], sgn[head][slot][m/32]
 *                          (one slot's planes contiguous; used for keys)
 *   TQ_LAYOUT_BLOCK32:     idx[head][slot/32][q][d] bit (slot%32),
 *                          sgn[head][slot/32][m]    bit (slot%32)
 *                          (32 slots share a word per coordinate; used for values)
 * Both: scl[head][slot][2] = fp16 bits of (||x||, ||r||); with the sketch off the
 * second entry is 0 and sgn may be NULL. */
typedef enum { TQ_LAYOUT_TOKEN_MAJOR = 0, TQ_LAYOUT_BLOCK32 = 1 } tq_layout;

enum {
  TQ_FLAG_NONFINITE_INPUT = 1u, /* a quantized vector held NaN or Inf          */
  TQ_FLAG_SCALE_OVERFLOW = 2u,  /* ||x|| or ||r|| > 65504: stored as 65504     */
  TQ_FLAG_OUT_OF_RANGE = 4u     /* a slot index fell outside the cache capacity;
                                   that vector/token was skipped              */
};

#define TQ_MAX_LEVELS 8

/* Lloyd-Max codebook of N(0, sigma^2) ([kiosk method]; [softpro 1.2] stage 1). */
typedef struct {
  int32_t bits_mse;                 /* b' in {1, 2, 3}                         */
  int32_t levels;                   /* L = 2^b'                                */
  double sigma;
  double centroid[TQ_MAX_LEVELS];   /* ascending, antisymmetric               */
  double boundary[TQ_MAX_LEVELS - 1]; /* boundary[k] = (centroid[k] + centroid[k+1]) / 2 */
  float centroid_f32[TQ_MAX_LEVELS];
  float boundary_f32[TQ_MAX_LEVELS - 1];
  /* Walsh expansion of the codebook over the bit-planes of the index:
   * with s_p = 2 b_p - 1 (b_p = bit p of the index),
   * centroid[i] = sum_{S subset of planes} walsh[S] * prod_{p in S} s_p(i),
   * walsh indexed by the subset's bit mask.  Only odd-size subsets are
   * non-zero for a symmetric codebook. */
  double walsh[TQ_MAX_LEVELS];
  double mse;                       /* expected squared error per coordinate   */
  int32_t iterations;
} tq_codebook;

/* Host, pure, reentrant.  Builds the b'-bit Lloyd-Max quantizer of
 * N(0, sigma^2) in float64 (alternating midpoint and conditional-mean
 * conditions until the centroids move by <= 1e-15 sigma), then makes it
 * exactly antisymmetric.  Returns TQ_ERR_INVALID_ARG for bits_mse outside
 * 1..3, sigma <= 0 or out == NULL; TQ_ERR_NO_CONVERGENCE after 100000 steps. */
int tq_build_codebook(int32_t bits_mse, double sigma, tq_codebook *out);

/* Host, pure, reentrant.  The b'-bit Lloyd-Max quantizer of the exact law of
 * one coordinate of a uniformly random unit vector in R^d, which is the law of
 * u = Pi x / ||x|| for a random rotation Pi: u^2 ~ Beta(1/2, (d-1)/2), density
 * (1 - u^2)^((d-3)/2) / B(1/2, (d-1)/2) on [-1, 1].  The method's theory is
 * stated with beta distributions (kiosknews.app "3 бита вместо 16", section
 * "Как работает TurboQuant"); the N(0, 1/d) law of tq_build_codebook is its
 * large-d limit.  Same iteration and
 * antisymmetrization as tq_build_codebook (stopping when the centroids move
 * by <= 1e-13 sigma), in absolute u units; sigma is set
 * to 1/sqrt(d) for reference and mse is the expected squared error per
 * coordinate under this law.  Returns TQ_ERR_INVALID_ARG for bits_mse outside
 * 1..3, d < 3 or out == NULL; TQ_ERR_NO_CONVERGENCE after 100000 steps. */
int tq_build_codebook_sphere(int32_t bits_mse, int32_t d, tq_codebook *out);

/* Per-tensor settings: b' index bits, and whether the 1-bit sign sketch plus
 * ||r|| is stored ([softpro 1.2] stage 2).  Total bits per value b = b' + sketch. */
typedef struct {
  int32_t bits_mse;                 /* b' in {1, 2, 3}                         */
  int32_t sketch;                   /* 1: sign sketch stored; 0: MSE only      */
  tq_codebook cb;                   /* built with sigma = 1/sqrt(d)            */
} tq_tensor_spec;

typedef struct {
  int32_t d;                        /* head dim: 64, 128 or 256                */
  int32_t m;                        /* sketch rows; must equal d               */
  int32_t n_kv_heads, n_q_heads;    /* n_q_heads a multiple of n_kv_heads      */
  const float *rot;                 /* device Pi [d][d], row-major, z = Pi x   */
  const float *proj;                /* device S [m][d], row-major              */
  const void *prep;                 /* device copy of the tq_prepare blob      */
  tq_tensor_spec k, v;              /* key and value settings                  */
} tq_config;

/* One packed cache (keys or values of one layer); caller-owned device memory.
 * Sizes: TOKEN_MAJOR idx = heads*capacity*b'*(d/32) words, sgn = heads*capacity*(m/32);
 *        BLOCK32     idx = heads*(capacity/32)*b'*d words,  sgn = heads*(capacity/32)*m;
 *        scl = heads*capacity*2 uint16.  capacity must be a multiple of 32. */
typedef struct {
  uint32_t *idx;
  uint32_t *sgn;
  uint16_t *scl;
  int64_t capacity;                 /* token slots per head                    */
  int32_t layout;                   /* tq_layout                               */
} tq_cache;

/* Host precomputation of the device-side matrices, in float64 then rounded:
 * Pi^T and S~^T = (S Pi^T)^T as fp32, and Pi, S~ split into bf16 hi/mid/lo
 * parts (hi + mid + lo reproduces the fp32 value exactly).  The caller copies
 * the blob to device memory and passes it as tq_config.prep.
 * tq_prepare_bytes returns 0 for unsupported sizes.  tq_prepare returns
 * TQ_ERR_INVALID_ARG for null pointers or m != d, TQ_ERR_UNSUPPORTED for d
 * other than 64/128/256. */
size_t tq_prepare_bytes(int32_t d, int32_t m);
int tq_prepare(const float *rot_host, const float *proj_host, int32_t d, int32_t m, void *blob_host);

/* Quantize and append ([softpro 1.2] stages 1 and 2; [kiosk python]).
 * k, v: device [batch][n_kv_heads][n_new][d] in dtype dt (either may be NULL
 * to skip that tensor).  Vector (b, h, t) is written to slot dst_token[b] + t
 * of head h of kc (keys) / vc (values).  dst_token: device int64 [batch].
 * The ranges [dst_token[b], dst_token[b] + n_new) of different b must not
 * overlap: overlapping writes race and leave either vector's record.  (A
 * ragged prefill is one call per sequence, or n_new padded into reserved slots.)
 * status: device uint32 (may be NULL) receiving TQ_FLAG_* bits.
 * dbg_scales: device fp32 [2][batch][n_kv_heads][n_new][2] or NULL; receives
 * the unrounded (||x||, ||r||) of each vector (tensor 0 = keys, 1 = values).
 * Slots outside [0, capacity) are skipped and flagged.  Errors:
 * TQ_ERR_INVALID_ARG (null config/caches for a given tensor, batch or n_new
 * < 0, misaligned pointers, inconsistent config), TQ_ERR_UNSUPPORTED,
 * TQ_ERR_LAUNCH.  batch * n_new == 0 enqueues nothing. */
int tq_quantize_kv(const tq_config *cfg, const void *k, const void *v, tq_dtype dt,
                   int32_t batch, int32_t n_new, const int64_t *dst_token,
                   const tq_cache *kc, const tq_cache *vc, uint32_t *status,
                   float *dbg_scales, hipStream_t stream);

/* Workspace bytes tq_decode_attention needs for this batch and longest length. */
size_t tq_decode_workspace_bytes(const tq_config *cfg, int32_t batch, int32_t max_len);

/* Decode attention over the packed caches (one new query per sequence and
 * query head).  The pages place the method's speed-up in decode, which reads
 * the compressed cache and so moves less data between memory and the GPU
 * (ast-softpro.ru, "Технология TurboQuant и её применение с локальными LLM",
 * section 1.3); the attention itself is not defined there, so the standard
 * scaled dot-product form is taken: out = softmax(q . k~ * sm_scale) . v~ over
 * every cached token of the sequence, with k~, v~ the vectors the records
 * encode (section 1.2: nu~ Pi^T c[idx] + sqrt(pi/2)/m rho~ S^T sgn) and query
 * head h reading kv head h / G, G = n_q_heads / n_kv_heads (any G <= 16; the
 * matrix-core kernels take G = 4 and 8 at d = 128 and 256, every other shape
 * runs the reference-grade kernels).
 * q: device [batch][n_q_heads][d] in dtype dt.  Sequence s occupies slots
 * [seq_start[s], seq_start[s] + seq_len[s]) of both caches (device int64
 * [batch] and int32 [batch]); max_len is the host-side bound on every seq_len
 * that sizes the launch and the workspace (a longer sequence is cut to its
 * first max_len tokens and flagged TQ_FLAG_OUT_OF_RANGE).  kc must be
 * TOKEN_MAJOR and vc BLOCK32 (TQ_ERR_UNSUPPORTED otherwise).  sm_scale 0
 * means 1/sqrt(d).  out: device fp32 [batch][n_q_heads][d].  A sequence of
 * length 0 yields zeros; a range outside the capacity is clipped and flagged
 * in *status (may be NULL).  workspace: device, >= tq_decode_workspace_bytes
 * bytes, caller-owned; its contents on entry do not matter.
 * Errors: TQ_ERR_INVALID_ARG, TQ_ERR_WORKSPACE, TQ_ERR_UNSUPPORTED (G > 16,
 * wrong layouts), TQ_ERR_LAUNCH. */
int tq_decode_attention(const tq_config *cfg, const void *q, tq_dtype dt, int32_t batch,
                        const int64_t *seq_start, const int32_t *seq_len, int32_t max_len,
                        const tq_cache *kc, const tq_cache *vc, float sm_scale, float *out,
                        uint32_t *status, void *workspace, size_t ws_bytes, hipStream_t stream);

/* Sparse V decode attention: tq_decode_attention whose value sum leaves out
 * the positions with low attention weight (kiosknews.app, "3 бита вместо 16:
 * разбираем TurboQuant и когда его реально стоит включать", section "Что
 * работает прямо сейчас и как попробовать", llama.cpp paragraph: decode skips
 * positions with low attention weights).  The page gives no rule; reading
 * taken: with M the head's largest score over the sequence, the value of
 * position t is left out when exp(s_t - M) < tau; the softmax normalizer keeps
 * every position, so out = sum over kept t of softmax(s)_t v~_t.  tau = 0 is
 * tq_decode_attention; tau = 1 keeps only the positions of the largest score.
 * Runs a first pass over the keys that records every split's largest score,
 * then the split pass, which skips the value products of 64-token tiles whose
 * values are all left out.  Same arguments, workspace and errors as
 * tq_decode_attention, plus TQ_ERR_INVALID_ARG for tau outside [0, 1] and
 * TQ_ERR_UNSUPPORTED for 0 < tau on shapes the matrix-core kernels do not take
 * (d other than 128 and 256, G other than 4 and 8, asymmetric codebooks). */
int tq_decode_attention_sparse_v(const tq_config *cfg, const void *q, tq_dtype dt, int32_t batch,
                                 const int64_t *seq_start, const int32_t *seq_len, int32_t max_len,
                                 const tq_cache *kc, const tq_cache *vc, float sm_scale, float tau, float *out,
                                 uint32_t *status, void *workspace, size_t ws_bytes, hipStream_t stream);

/* Bytes of the fixed device scratch behind tq_decode_attention_noalloc (per device). */
#define TQ_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* tq_decode_attention without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, kernels and outputs as
 * tq_decode_attention; the workspace is a fixed TQ_NOALLOC_SCRATCH_BYTES array
 * inside the library, one per device, held from when the library's code is
 * loaded on the device until the process ends.  The call allocates nothing.
 * Every call on a device shares that device's array: calls that overlap on
 * one device (other streams, other threads) race and must be serialized by the
 * caller.  Returns TQ_ERR_WORKSPACE when tq_decode_workspace_bytes(cfg, batch,
 * max_len) exceeds the array (for example 256 query heads over 128K tokens need
 * about 35 MB, 2,048 query heads over 16K tokens about 38 MB), TQ_ERR_LAUNCH if
 * the array's address cannot be found on the current device, and otherwise
 * what tq_decode_attention returns. */
int tq_decode_attention_noalloc(const tq_config *cfg, const void *q, tq_dtype dt, int32_t batch,
                                const int64_t *seq_start, const int32_t *seq_len, int32_t max_len,
                                const tq_cache *kc, const tq_cache *vc, float sm_scale, float *out,
                                uint32_t *status, hipStream_t stream);

/* Workspace bytes tq_score_keys needs for n_q queries over at most max_n keys. */
size_t tq_score_workspace_bytes(const tq_config *cfg, int32_t n_q, int32_t max_n);

/* Inner-product scores of n_q queries against packed keys: the compressed
 * vectors as a search index (ast-softpro.ru, "Технология TurboQuant и её
 * применение с локальными LLM", section 6.4 and FAQ: vector search in RAG
 * systems).  scores[j][i] = <q_j, k~_i> for the key in slot start + i of head
 * kv_head of kc, i < n, where k~ is the vector the record encodes
 * (nu~ Pi^T c[idx] + sqrt(pi/2)/m rho~ S^T sgn, section 1.2) -- the estimator
 * decode attention scores, without a softmax scale.  q: device
 * [n_q][d] in dtype dt, n_q a positive multiple of 8; kc: TOKEN_MAJOR.
 * scores: device fp32 [n_q][n] (row stride n).  A range past the capacity
 * is rejected (TQ_ERR_INVALID_ARG); d other than 128 or 256 and an
 * asymmetric codebook give TQ_ERR_UNSUPPORTED.  workspace: device,
 * >= tq_score_workspace_bytes.  Enqueues on stream and returns. */
int tq_score_keys(const tq_config *cfg, const void *q, tq_dtype dt, int32_t n_q, const tq_cache *kc,
                  int32_t kv_head, int64_t start, int32_t n, float *scores, uint32_t *status,
                  void *workspace, size_t ws_bytes, hipStream_t stream);

/* Static string for a tq_status value. */
const char *tq_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* TQ_H */
