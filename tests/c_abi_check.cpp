// Standalone use of libwaveprune from C++, no torch: the caller allocates
// with hipMalloc, builds the cutoff table on the host, runs RoPE, prefill and
// decode through the C ABI, and checks
//  * that the decode of the last token (query position n-1, keys 0..n-1 of
//    the cache) reproduces the prefill's last row, which attends the same keys
//    under the same rule;
//  * that invalid arguments come back as negative status codes with a message,
//    before anything is enqueued.
// Prints one line and exits 0 on success, 1 on failure.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "waveprune.h"

namespace {

uint16_t to_bf16(float f) {   // nearest even
  uint32_t u;
  std::memcpy(&u, &f, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
float from_bf16(uint16_t h) {
  const uint32_t u = (uint32_t)h << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}
// deterministic uniform(-1, 1) values
float next_val(uint64_t& s) {
  s = s * 6364136223846793005ull + 1442695040888963407ull;
  return (float)((s >> 40) & 0xffffff) / 8388608.0f - 1.0f;
}

#define CHECK_HIP(x)                                                             \
  do {                                                                           \
    if ((x) != hipSuccess) {                                                     \
      std::printf("c_abi_check FAIL: %s at line %d\n", #x, __LINE__);           \
      return 1;                                                                  \
    }                                                                            \
  } while (0)

}  // namespace

int main() {
  const int B = 1, n = 300, Hq = 4, Hkv = 2, d = 128, G = 16;
  const double theta = 300.0;
  int32_t cut[d / G];
  if (wp_group_cutoffs(theta, d, G, 1.0, cut, d / G) != WP_OK) {
    std::printf("c_abi_check FAIL: wp_group_cutoffs: %s\n", wp_last_error());
    return 1;
  }
  // raw q, k, v [B, n, H, d] bf16
  uint64_t seed = 12345;
  std::vector<uint16_t> hq((size_t)n * Hq * d), hk((size_t)n * Hkv * d), hv((size_t)n * Hkv * d);
  for (auto& x : hq) x = to_bf16(next_val(seed));
  for (auto& x : hk) x = to_bf16(next_val(seed));
  for (auto& x : hv) x = to_bf16(next_val(seed));
  void *q, *k, *v, *qr, *kr, *o, *od, *ws;
  CHECK_HIP(hipMalloc(&q, hq.size() * 2));
  CHECK_HIP(hipMalloc(&k, hk.size() * 2));
  CHECK_HIP(hipMalloc(&v, hv.size() * 2));
  CHECK_HIP(hipMalloc(&qr, hq.size() * 2));
  CHECK_HIP(hipMalloc(&kr, hk.size() * 2));
  CHECK_HIP(hipMalloc(&o, hq.size() * 2));
  CHECK_HIP(hipMalloc(&od, (size_t)B * Hq * d * 2));
  const size_t ws_bytes = wp_decode_workspace_size(B, n, Hq, Hkv, d, 0);
  CHECK_HIP(hipMalloc(&ws, ws_bytes));
  int32_t *cl, *qp;
  CHECK_HIP(hipMalloc(&cl, sizeof(int32_t) * B));
  CHECK_HIP(hipMalloc(&qp, sizeof(int32_t) * B));
  CHECK_HIP(hipMemcpy(q, hq.data(), hq.size() * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(k, hk.data(), hk.size() * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(v, hv.data(), hv.size() * 2, hipMemcpyHostToDevice));
  const int32_t len = n, pos = n - 1;
  CHECK_HIP(hipMemcpy(cl, &len, sizeof(len), hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(qp, &pos, sizeof(pos), hipMemcpyHostToDevice));
  hipStream_t s;
  CHECK_HIP(hipStreamCreate(&s));

  // strides in elements
  const int64_t sq[3] = {(int64_t)n * Hq * d, (int64_t)Hq * d, d};
  const int64_t skv[3] = {(int64_t)n * Hkv * d, (int64_t)Hkv * d, d};
  int st;
  if ((st = wp_rope_apply(q, WP_DTYPE_BF16, qr, B, n, Hq, d, sq, sq, nullptr, theta, 1.0, s)) != WP_OK ||
      (st = wp_rope_apply(k, WP_DTYPE_BF16, kr, B, n, Hkv, d, skv, skv, nullptr, theta, 1.0, s)) != WP_OK) {
    std::printf("c_abi_check FAIL: wp_rope_apply %d: %s\n", st, wp_last_error());
    return 1;
  }
  const int64_t sp[12] = {sq[0], sq[1], sq[2], skv[0], skv[1], skv[2], skv[0], skv[1], skv[2], sq[0], sq[1], sq[2]};
  if ((st = wp_prefill(qr, kr, v, o, nullptr, B, n, Hq, Hkv, d, sp, cut, G, 0, nullptr, s)) != WP_OK) {
    std::printf("c_abi_check FAIL: wp_prefill %d: %s\n", st, wp_last_error());
    return 1;
  }
  // decode: the query is the last token's rotated q, the cache the rotated K
  const char* q_last = (const char*)qr + (size_t)(n - 1) * Hq * d * 2;
  const int64_t sd[10] = {(int64_t)Hq * d, d, skv[0], skv[1], skv[2], skv[0], skv[1], skv[2], (int64_t)Hq * d, d};
  if ((st = wp_decode(q_last, kr, v, od, cl, qp, B, n, Hq, Hkv, d, sd, cut, G, 0, ws, ws_bytes, 0, nullptr, s)) !=
      WP_OK) {
    std::printf("c_abi_check FAIL: wp_decode %d: %s\n", st, wp_last_error());
    return 1;
  }
  // invalid calls: status codes and messages, nothing enqueued
  const int e1 = wp_prefill(qr, kr, v, o, nullptr, B, n, Hq, Hkv, 96, sp, cut, G, 0, nullptr, s);
  const bool msg1 = std::strlen(wp_last_error()) > 0;
  const int e2 = wp_decode(q_last, kr, v, od, cl, qp, B, n, Hq, Hkv, d, sd, cut, G, 0, ws, 16, 0, nullptr, s);
  const int e3 = wp_prefill(qr, kr, v, o, nullptr, B, n, 3, Hkv, d, sp, cut, G, 0, nullptr, s);
  CHECK_HIP(hipStreamSynchronize(s));

  std::vector<uint16_t> ho(hq.size()), hod((size_t)Hq * d);
  CHECK_HIP(hipMemcpy(ho.data(), o, ho.size() * 2, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(hod.data(), od, hod.size() * 2, hipMemcpyDeviceToHost));
  double maxd = 0.0, maxv = 0.0;
  for (int h = 0; h < Hq; ++h)
    for (int c = 0; c < d; ++c) {
      const float a = from_bf16(ho[((size_t)(n - 1) * Hq + h) * d + c]);
      const float b = from_bf16(hod[(size_t)h * d + c]);
      maxd = std::fmax(maxd, std::fabs((double)a - b));
      maxv = std::fmax(maxv, std::fabs((double)a));
    }
  const bool ok = maxd <= 2e-2 && maxv > 0.0 && e1 == WP_ERR_UNSUPPORTED && msg1 && e2 == WP_ERR_WORKSPACE &&
                  e3 == WP_ERR_SHAPE;
  std::printf("c_abi_check %s: decode vs prefill last row max-abs %.3e (max |o| %.3f); status codes %d %d %d (%s)\n",
              ok ? "OK" : "FAIL", maxd, maxv, e1, e2, e3, wp_version());
  for (void* p : {q, k, v, qr, kr, o, od, ws}) (void)hipFree(p);
  (void)hipFree(cl);
  (void)hipFree(qp);
  (void)hipStreamDestroy(s);
  return ok ? 0 : 1;
}
