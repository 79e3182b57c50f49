// Drives every host-side path of libtq's C ABI (codebooks, tq_prepare, argument
// validation, workspace plans, the dispatch to the launchers) for a build of
// tq_host.cpp under AddressSanitizer and UndefinedBehaviorSanitizer.  Device
// pointers are host buffers here: the host code only checks and forwards them.
// Exit status 0 when every expectation holds; the sanitizers abort otherwise.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "tq.h"

namespace tq {
extern int g_launches;
}

static int failures = 0;
#define EXPECT(cond)                                                     \
  do {                                                                   \
    if (!(cond)) {                                                       \
      std::fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                        \
    }                                                                    \
  } while (0)

// 16-byte aligned host storage standing in for device buffers.
struct Buf {
  std::vector<unsigned char> v;
  explicit Buf(size_t n) : v(n + 16) {}
  void *p() {
    auto a = reinterpret_cast<uintptr_t>(v.data());
    return reinterpret_cast<void *>((a + 15) & ~uintptr_t(15));
  }
};

static void codebooks() {
  for (int b = 1; b <= 3; ++b) {
    tq_codebook cb;
    EXPECT(tq_build_codebook(b, 1.0 / std::sqrt(128.0), &cb) == TQ_OK);
    EXPECT(cb.levels == (1 << b));
    for (int i = 0; i < cb.levels; ++i) EXPECT(cb.centroid[i] == -cb.centroid[cb.levels - 1 - i]);
    for (int d : {3, 8, 64, 128, 256}) {
      tq_codebook cs;
      EXPECT(tq_build_codebook_sphere(b, d, &cs) == TQ_OK);
      EXPECT(cs.mse > 0.0);
    }
  }
  tq_codebook cb;
  EXPECT(tq_build_codebook(0, 1.0, &cb) == TQ_ERR_INVALID_ARG);
  EXPECT(tq_build_codebook(4, 1.0, &cb) == TQ_ERR_INVALID_ARG);
  EXPECT(tq_build_codebook(2, 0.0, &cb) == TQ_ERR_INVALID_ARG);
  EXPECT(tq_build_codebook(2, 1.0, nullptr) == TQ_ERR_INVALID_ARG);
  EXPECT(tq_build_codebook_sphere(2, 2, &cb) == TQ_ERR_INVALID_ARG);
  for (int s = -6; s <= 1; ++s) EXPECT(tq_status_string(s) != nullptr);
}

struct Setup {
  int d, hkv, hq, bits;
  Buf rot, proj, prep;
  tq_config cfg{};
  Setup(int d_, int hkv_, int hq_, int bits_)
      : d(d_), hkv(hkv_), hq(hq_), bits(bits_), rot(size_t(d_) * d_ * 4), proj(size_t(d_) * d_ * 4),
        prep(tq_prepare_bytes(d_, d_)) {
    std::vector<float> r(size_t(d) * d), s(size_t(d) * d);
    unsigned x = 12345u;
    for (auto &e : r) e = (x = x * 1664525u + 1013904223u) / 4294967296.0f - 0.5f;
    for (auto &e : s) e = (x = x * 1664525u + 1013904223u) / 4294967296.0f - 0.5f;
    EXPECT(tq_prepare(r.data(), s.data(), d, d, prep.p()) == TQ_OK);
    cfg.d = d;
    cfg.m = d;
    cfg.n_kv_heads = hkv;
    cfg.n_q_heads = hq;
    cfg.rot = static_cast<const float *>(rot.p());
    cfg.proj = static_cast<const float *>(proj.p());
    cfg.prep = prep.p();
    for (tq_tensor_spec *t : {&cfg.k, &cfg.v}) {
      t->bits_mse = bits;
      t->sketch = 1;
      EXPECT(tq_build_codebook(bits, 1.0 / std::sqrt(double(d)), &t->cb) == TQ_OK);
    }
  }
};

struct Cache {
  Buf idx, sgn, scl;
  tq_cache c{};
  Cache(int heads, int64_t cap, int d, int bits, int layout)
      : idx(size_t(heads) * cap * bits * d / 8), sgn(size_t(heads) * cap * d / 8), scl(size_t(heads) * cap * 4) {
    c.idx = static_cast<uint32_t *>(idx.p());
    c.sgn = static_cast<uint32_t *>(sgn.p());
    c.scl = static_cast<uint16_t *>(scl.p());
    c.capacity = cap;
    c.layout = layout;
  }
};

static void prepare_errors() {
  EXPECT(tq_prepare_bytes(96, 96) == 0);
  std::vector<float> m(64 * 64, 0.0f);
  Buf blob(tq_prepare_bytes(64, 64));
  EXPECT(tq_prepare(nullptr, m.data(), 64, 64, blob.p()) == TQ_ERR_INVALID_ARG);
  EXPECT(tq_prepare(m.data(), m.data(), 64, 32, blob.p()) == TQ_ERR_INVALID_ARG);
}

static void quantize_and_decode(int d, int hkv, int hq, int bits) {
  Setup S(d, hkv, hq, bits);
  const int B = 3, n_new = 5;
  const int64_t cap = 256;
  Cache kc(hkv, cap, d, bits, TQ_LAYOUT_TOKEN_MAJOR), vc(hkv, cap, d, bits, TQ_LAYOUT_BLOCK32);
  Buf x(size_t(B) * hkv * n_new * d * 4), dst(B * 8), st(4), dbg(size_t(2) * B * hkv * n_new * 2 * 4);
  auto *dstp = static_cast<int64_t *>(dst.p());
  for (int b = 0; b < B; ++b) dstp[b] = 64 * b;
  const int before = tq::g_launches;
  EXPECT(tq_quantize_kv(&S.cfg, x.p(), x.p(), TQ_BF16, B, n_new, dstp, &kc.c, &vc.c,
                        static_cast<uint32_t *>(st.p()), static_cast<float *>(dbg.p()), nullptr) == TQ_OK);
  EXPECT(tq::g_launches > before);
  EXPECT(tq_quantize_kv(&S.cfg, x.p(), nullptr, TQ_F32, B, 1, dstp, &kc.c, nullptr, nullptr, nullptr, nullptr) == TQ_OK);
  EXPECT(tq_quantize_kv(&S.cfg, x.p(), x.p(), TQ_BF16, B, 0, dstp, &kc.c, &vc.c, nullptr, nullptr, nullptr) == TQ_OK);
  EXPECT(tq_quantize_kv(&S.cfg, x.p(), x.p(), TQ_BF16, -1, 1, dstp, &kc.c, &vc.c, nullptr, nullptr, nullptr) ==
         TQ_ERR_INVALID_ARG);
  EXPECT(tq_quantize_kv(&S.cfg, static_cast<char *>(x.p()) + 4, nullptr, TQ_BF16, B, 1, dstp, &kc.c, nullptr,
                        nullptr, nullptr, nullptr) == TQ_ERR_INVALID_ARG);
  for (int bad : {7, -1, 0x7FFFFFFF})
    EXPECT(tq_quantize_kv(&S.cfg, x.p(), x.p(), static_cast<tq_dtype>(bad), B, 1, dstp, &kc.c, &vc.c, nullptr,
                          nullptr, nullptr) == TQ_ERR_INVALID_ARG);

  // decode
  const int32_t max_len = 200;
  const size_t wsb = tq_decode_workspace_bytes(&S.cfg, B, max_len);
  EXPECT(wsb > 0);
  Buf ws(wsb), q(size_t(B) * hq * d * 4), out(size_t(B) * hq * d * 4), lens(B * 4);
  auto *lp = static_cast<int32_t *>(lens.p());
  for (int b = 0; b < B; ++b) lp[b] = 100 + 50 * b;
  auto *outp = static_cast<float *>(out.p());
  EXPECT(tq_decode_attention(&S.cfg, q.p(), TQ_BF16, B, dstp, lp, max_len, &kc.c, &vc.c, 0.0f, outp,
                             static_cast<uint32_t *>(st.p()), ws.p(), wsb, nullptr) == TQ_OK);
  EXPECT(tq_decode_attention_sparse_v(&S.cfg, q.p(), TQ_BF16, B, dstp, lp, max_len, &kc.c, &vc.c, 0.0f, 1e-3f,
                                      outp, nullptr, ws.p(), wsb, nullptr) ==
         ((d == 128 || d == 256) && (hq / hkv == 4 || hq / hkv == 8) ? TQ_OK : TQ_ERR_UNSUPPORTED));
  EXPECT(tq_decode_attention(&S.cfg, q.p(), TQ_BF16, B, dstp, lp, max_len, &kc.c, &vc.c, 0.0f, outp, nullptr,
                             ws.p(), wsb - 1, nullptr) == TQ_ERR_WORKSPACE);
  EXPECT(tq_decode_attention(&S.cfg, q.p(), TQ_BF16, B, dstp, lp, max_len, &vc.c, &kc.c, 0.0f, outp, nullptr,
                             ws.p(), wsb, nullptr) == TQ_ERR_UNSUPPORTED);
  EXPECT(tq_decode_attention(&S.cfg, q.p(), TQ_BF16, B, dstp, lp, max_len, &kc.c, &vc.c, -1.0f, outp, nullptr,
                             ws.p(), wsb, nullptr) == TQ_ERR_INVALID_ARG);
  EXPECT(tq_decode_attention(&S.cfg, q.p(), TQ_BF16, B, dstp, lp, max_len, &kc.c, &vc.c, 0.0f, outp, nullptr,
                             ws.p(), wsb, nullptr) == TQ_OK);

  // key scoring
  if (d == 128 || d == 256) {
    for (int nq : {8, 16, 24}) {
      const size_t sb = tq_score_workspace_bytes(&S.cfg, nq, 150);
      EXPECT(sb > 0);
      Buf sw(sb), qs(size_t(nq) * d * 4), sc(size_t(nq) * 150 * 4);
      EXPECT(tq_score_keys(&S.cfg, qs.p(), TQ_BF16, nq, &kc.c, 0, 3, 150, static_cast<float *>(sc.p()), nullptr,
                           sw.p(), sb, nullptr) == TQ_OK);
      EXPECT(tq_score_keys(&S.cfg, qs.p(), TQ_BF16, nq, &kc.c, hkv, 3, 150, static_cast<float *>(sc.p()), nullptr,
                           sw.p(), sb, nullptr) == TQ_ERR_INVALID_ARG);
    }
    EXPECT(tq_score_workspace_bytes(&S.cfg, 12, 10) == 0);
  }
}

int main() {
  codebooks();
  prepare_errors();
  quantize_and_decode(128, 8, 64, 2);  // matrix-core paths, G = 8
  quantize_and_decode(128, 8, 32, 3);  // G = 4
  quantize_and_decode(256, 4, 16, 1);  // d = 256
  quantize_and_decode(128, 2, 12, 2);  // G = 6: reference-grade decode
  quantize_and_decode(64, 2, 2, 2);    // d = 64: reference-grade kernels
  if (failures) {
    std::fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  std::printf("host paths ok (%d launches)\n", tq::g_launches);
  return 0;
}
