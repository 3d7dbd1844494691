// Sanitizer run of libwaveprune's host code on the CPU: the C ABI (api.hip,
// built with AddressSanitizer and UndefinedBehaviorSanitizer) linked against
// host stand-ins of the kernel launchers (launch_stubs.cpp) that touch the
// first and last byte of every range a launch would address.  Host memory
// stands in for device memory.  Exercises: cutoff tables, the host tile
// classifier, tiling queries, compact-store geometry, every entry point on
// valid shapes (contiguous and strided, ragged), and the validation errors.
// Prints "host_check ok <n>" and exits 0 on success.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "../../include/waveprune.h"

extern "C" long long wp_host_check_touched();

static int g_fail = 0;
#define EXPECT(cond)                                                             \
  do {                                                                           \
    if (!(cond)) {                                                               \
      fprintf(stderr, "FAIL %s:%d: %s (%s)\n", __FILE__, __LINE__, #cond, wp_last_error()); \
      ++g_fail;                                                                  \
    }                                                                            \
  } while (0)

// a host allocation of exactly n bytes with a 256-byte aligned base (the
// sanitizer's redzone starts right after the last byte)
struct Buf {
  unsigned char* p = nullptr;
  explicit Buf(size_t n) {
    void* q = nullptr;
    if (posix_memalign(&q, 256, n ? n : 1)) abort();
    p = static_cast<unsigned char*>(q);
    memset(p, 0, n);
  }
  ~Buf() { free(p); }
  Buf(const Buf&) = delete;
  Buf& operator=(const Buf&) = delete;
};

static void cutoffs_and_tiles() {
  const int dims[2] = {64, 128};
  for (int d : dims)
    for (int G : {2, 4, 8, 16, 32}) {
      const int ng = d / G;
      std::vector<int32_t> cut(ng);
      for (double th : {10.0, 1e4, 1e6, 1e12})
        for (double s : {1.0, 4.0}) EXPECT(wp_group_cutoffs(th, d, G, s, cut.data(), ng) == WP_OK);
      for (int g = 1; g < ng; ++g) EXPECT(cut[g] >= cut[g - 1]);
      std::vector<int64_t> cnt(3 * ng + 1);
      for (int n : {1, 31, 32, 33, 64, 100, 4096})
        EXPECT(wp_prefill_tile_counts(n, d, G, cut.data(), cnt.data()) == WP_OK);
      for (int L : {0, 1, 33, 5000}) EXPECT(wp_decode_tile_counts(L + 3, L, d, G, cut.data(), cnt.data()) == WP_OK);
      int32_t bm, bn;
      EXPECT(wp_prefill_tiling(d, G, &bm, &bn) == WP_OK && wp_decode_tiling(d, G, &bn) == WP_OK);
      std::vector<double> f(d / 2);
      for (int c = 0; c < d / 2; ++c) f[c] = pow(1e4, -2.0 * c / d);
      EXPECT(wp_cutoffs_from_freqs(f.data(), d / 2, 2.0, d / 4, G, cut.data(), ng) == WP_OK);
      EXPECT(wp_cutoffs_from_freqs(f.data(), d / 2, INFINITY, 0, G, cut.data(), ng) == WP_OK);
    }
  // errors
  int32_t cut8[8];
  EXPECT(wp_group_cutoffs(-1.0, 128, 16, 1.0, cut8, 8) == WP_ERR_ARG);
  EXPECT(wp_group_cutoffs(1e4, 128, 16, NAN, cut8, 8) == WP_ERR_ARG);
  EXPECT(wp_group_cutoffs(1e4, 128, 12, 1.0, cut8, 8) == WP_ERR_SHAPE);
  EXPECT(wp_group_cutoffs(1e4, 128, 16, 1.0, cut8, 7) == WP_ERR_SHAPE);
  EXPECT(wp_group_cutoffs(1e4, 128, 16, 1.0, nullptr, 8) == WP_ERR_NULL);
  int64_t cnt[25];
  EXPECT(wp_prefill_tile_counts(0, 128, 16, cut8, cnt) == WP_ERR_SHAPE);
  EXPECT(wp_prefill_tile_counts(10, 96, 16, cut8, cnt) == WP_ERR_UNSUPPORTED);
  int32_t bad[8] = {5, 4, 9, 9, 9, 9, 9, 9};
  EXPECT(wp_prefill_tile_counts(10, 128, 16, bad, cnt) == WP_ERR_ARG);
  EXPECT(wp_decode_tile_counts(3, 10, 128, 16, cut8, cnt) == WP_ERR_ARG);
}

static void rope() {
  const int B = 2, n = 37, H = 3, d = 128;
  Buf x(sizeof(float) * B * n * H * d), y(2 * B * n * H * d), pos(8 * B);
  const int64_t sx[3] = {n * H * d, H * d, d};
  EXPECT(wp_rope_apply(x.p, WP_DTYPE_F32, y.p, B, n, H, d, sx, sx, (int64_t*)pos.p, 1e4, 1.0, nullptr) == WP_OK);
  EXPECT(wp_rope_apply(y.p, WP_DTYPE_BF16, y.p, B, n, H, d, sx, sx, nullptr, 1e4, 4.0, nullptr) == WP_OK);
  // a head view of a wider tensor (stride 5 heads, one head used)
  Buf w(2 * B * n * 5 * d);
  const int64_t sw[3] = {n * 5 * d, 5 * d, d};
  EXPECT(wp_rope_apply(w.p + 2 * 4 * d, WP_DTYPE_BF16, w.p + 2 * 4 * d, B, n, 1, d, sw, sw, nullptr, 1e6, 1.0,
                       nullptr) == WP_OK);
  EXPECT(wp_rope_apply(x.p, 7, y.p, B, n, H, d, sx, sx, nullptr, 1e4, 1.0, nullptr) == WP_ERR_ARG);
  EXPECT(wp_rope_apply(x.p, WP_DTYPE_F32, x.p, B, n, H, d, sx, sx, nullptr, 1e4, 1.0, nullptr) == WP_ERR_ARG);
  EXPECT(wp_rope_apply(x.p + 2, WP_DTYPE_F32, y.p, B, n, H, d, sx, sx, nullptr, 1e4, 1.0, nullptr) == WP_ERR_ALIGN);
}

static void prefill_and_backward() {
  for (int d : {64, 128})
    for (int G : {2, 16, 32}) {
      const int B = 2, n = 77, Hq = 6, Hkv = 2, ng = d / G;
      std::vector<int32_t> cut(ng);
      EXPECT(wp_group_cutoffs(300.0, d, G, 1.0, cut.data(), ng) == WP_OK);
      const size_t qe = (size_t)B * n * Hq * d, ke = (size_t)B * n * Hkv * d;
      Buf q(2 * qe), k(2 * ke), v(2 * ke), o(2 * qe), lse(4 * B * Hq * n), cnt(8 * (3 * ng + 1));
      const int64_t st[12] = {n * Hq * d, Hq * d, d, n * Hkv * d, Hkv * d, d, n * Hkv * d, Hkv * d, d,
                              n * Hq * d, Hq * d, d};
      EXPECT(wp_prefill(q.p, k.p, v.p, o.p, (float*)lse.p, B, n, Hq, Hkv, d, st, cut.data(), G, WP_FLAG_COUNT,
                        (int64_t*)cnt.p, nullptr) == WP_OK);
      EXPECT(wp_prefill(q.p, k.p, v.p, o.p, nullptr, B, n, Hq, Hkv, d, st, nullptr, G, WP_FLAG_DENSE, nullptr,
                        nullptr) == WP_OK);
      EXPECT(wp_prefill(q.p, k.p, v.p, o.p, nullptr, B, n, Hq, Hkv, d, st, cut.data(), G, WP_FLAG_MFMA16, nullptr,
                        nullptr) == ((d == 128 && G == 32) ? WP_OK : WP_ERR_UNSUPPORTED));
      // packed QKV projection output [B, n, Hq + 2 Hkv, d]
      const int Ht = Hq + 2 * Hkv;
      Buf qkv(2 * (size_t)B * n * Ht * d);
      const int64_t sp[12] = {n * Ht * d, Ht * d, d, n * Ht * d, Ht * d, d, n * Ht * d, Ht * d, d,
                              n * Hq * d, Hq * d, d};
      EXPECT(wp_prefill(qkv.p, qkv.p + 2 * Hq * d, qkv.p + 2 * (Hq + Hkv) * d, o.p, nullptr, B, n, Hq, Hkv, d, sp,
                        cut.data(), G, 0, nullptr, nullptr) == WP_OK);
      // backward
      Buf dout(2 * qe), dq(2 * qe), dk(2 * ke), dv(2 * ke);
      const size_t ws = wp_prefill_backward_workspace_size(B, n, Hq);
      Buf wsb(ws);
      int64_t sb[24];
      for (int t = 0; t < 8; ++t) {
        const bool qh = (t == 0 || t == 3 || t == 4 || t == 5);
        const int H = qh ? Hq : Hkv;
        sb[3 * t] = (int64_t)n * H * d;
        sb[3 * t + 1] = (int64_t)H * d;
        sb[3 * t + 2] = d;
      }
      if (G >= 2)
        EXPECT(wp_prefill_backward(q.p, k.p, v.p, o.p, dout.p, (float*)lse.p, dq.p, dk.p, dv.p, B, n, Hq, Hkv, d, sb,
                                   cut.data(), G, 0, wsb.p, ws, nullptr) == WP_OK);
      EXPECT(wp_prefill_backward(q.p, k.p, v.p, o.p, dout.p, (float*)lse.p, dq.p, dk.p, dv.p, B, n, Hq, Hkv, d, sb,
                                 cut.data(), G, 0, wsb.p, ws - 8, nullptr) == WP_ERR_WORKSPACE);
      // errors
      EXPECT(wp_prefill(q.p, k.p, v.p, o.p, nullptr, B, n, 5, Hkv, d, st, cut.data(), G, 0, nullptr, nullptr) ==
             WP_ERR_SHAPE);
      EXPECT(wp_prefill(q.p, k.p, v.p, o.p, nullptr, B, n, Hq, Hkv, d, st, cut.data(), G, 8, nullptr, nullptr) ==
             WP_ERR_ARG);
      EXPECT(wp_prefill(q.p, k.p, v.p, o.p, nullptr, B, n, Hq, Hkv, d, st, cut.data(), G, WP_FLAG_COUNT, nullptr,
                        nullptr) == WP_ERR_NULL);
    }
}

static void decode_paths() {
  for (int d : {64, 128})
    for (int G : {2, 16, 32}) {
      const int B = 3, Lmax = 300, Hq = 40, Hkv = 2, ng = d / G;   // 20 query heads per kv head: two passes
      std::vector<int32_t> cut(ng);
      EXPECT(wp_group_cutoffs(100.0, d, G, 1.0, cut.data(), ng) == WP_OK);
      Buf q(2 * B * Hq * d), o(2 * B * Hq * d), kc(2 * (size_t)B * Lmax * Hkv * d), vc(2 * (size_t)B * Lmax * Hkv * d);
      Buf cl(4 * B), qp(4 * B), cnt(8 * (3 * ng + 1));
      const int32_t lens[3] = {300, 0, 17};
      memcpy(cl.p, lens, sizeof(lens));
      const int32_t pos[3] = {300, 5, 16};
      memcpy(qp.p, pos, sizeof(pos));
      const int64_t st[10] = {Hq * d, d, Lmax * Hkv * d, Hkv * d, d, Lmax * Hkv * d, Hkv * d, d, Hq * d, d};
      for (int S : {0, 1, 7}) {
        const size_t ws = wp_decode_workspace_size(B, Lmax, Hq, Hkv, d, S);
        Buf w(ws);
        EXPECT(wp_decode(q.p, kc.p, vc.p, o.p, (int32_t*)cl.p, (int32_t*)qp.p, B, Lmax, Hq, Hkv, d, st, cut.data(), G,
                         S, w.p, ws, WP_FLAG_COUNT, (int64_t*)cnt.p, nullptr) == WP_OK);
        EXPECT(wp_decode(q.p, kc.p, vc.p, o.p, (int32_t*)cl.p, (int32_t*)qp.p, B, Lmax, Hq, Hkv, d, st, cut.data(), G,
                         S, w.p, ws - 1, 0, nullptr, nullptr) == WP_ERR_WORKSPACE);
        EXPECT(wp_decode_noalloc(q.p, kc.p, vc.p, o.p, (int32_t*)cl.p, (int32_t*)qp.p, B, Lmax, Hq, Hkv, d, st,
                                 cut.data(), G, S, 0, nullptr, nullptr) == WP_OK);
      }
      EXPECT(wp_decode_noalloc(q.p, kc.p, vc.p, o.p, (int32_t*)cl.p, (int32_t*)qp.p, 4000, Lmax, 64, Hkv, d, st,
                               cut.data(), G, 64, 0, nullptr, nullptr) == WP_ERR_WORKSPACE);
      if (G < 16) continue;
      // compact K store
      std::vector<int32_t> caps(ng);
      std::vector<int64_t> offs(ng + 1);
      EXPECT(wp_kcache_layout(Lmax, d, G, cut.data(), caps.data(), offs.data()) == WP_OK);
      const int64_t se = offs[ng];
      Buf store(2 * (size_t)B * Hkv * se), p0(4 * B);
      const int32_t zero[3] = {0, 0, 0};
      memcpy(p0.p, zero, sizeof(zero));
      const int64_t sk[3] = {Lmax * Hkv * d, Hkv * d, d};
      const int64_t ss[2] = {Hkv * se, se};
      EXPECT(wp_kcache_append(kc.p, B, Lmax, Hkv, d, sk, (int32_t*)p0.p, store.p, ss, Lmax, cut.data(), G, nullptr) ==
             WP_OK);
      const int64_t st9[9] = {Hq * d, d, Hkv * se, se, Lmax * Hkv * d, Hkv * d, d, Hq * d, d};
      const size_t ws = wp_decode_workspace_size(B, Lmax, Hq, Hkv, d, 0);
      Buf w(ws);
      EXPECT(wp_decode_kcache(q.p, store.p, vc.p, o.p, (int32_t*)cl.p, (int32_t*)qp.p, B, Lmax, Hq, Hkv, d, st9,
                              cut.data(), G, 0, w.p, ws, 0, nullptr, nullptr) == WP_OK);
      const int64_t ss_small[2] = {Hkv * se, se - 8};
      EXPECT(wp_kcache_append(kc.p, B, Lmax, Hkv, d, sk, (int32_t*)p0.p, store.p, ss_small, Lmax, cut.data(), G,
                              nullptr) == WP_ERR_SHAPE);
    }
}

// A planted mistake for the harness itself: K one element shorter than the
// shape says.  The launch stand-in's touch of the last key row must then be
// reported by AddressSanitizer (the test expects this run to fail).
static void undersized_k() {
  const int n = 50, H = 1, d = 64, G = 16;
  int32_t cut[4];
  wp_group_cutoffs(1e4, d, G, 1.0, cut, 4);
  Buf q(2 * n * H * d), k(2 * n * H * d - 2), v(2 * n * H * d), o(2 * n * H * d);
  const int64_t st[12] = {H * d, H * d, d, H * d, H * d, d, H * d, H * d, d, H * d, H * d, d};
  wp_prefill(q.p, k.p, v.p, o.p, nullptr, 1, n, H, H, d, st, cut, G, 0, nullptr, nullptr);
}

int main(int argc, char** argv) {
  if (argc > 1 && strcmp(argv[1], "undersized") == 0) {
    undersized_k();
    printf("host_check undersized: not reported\n");
    return 0;
  }
  cutoffs_and_tiles();
  rope();
  prefill_and_backward();
  decode_paths();
  printf("host_check %s %lld\n", g_fail ? "FAILED" : "ok", wp_host_check_touched());
  return g_fail ? 1 : 0;
}
