// libwaveprune C ABI: argument validation, the cutoff table, the host tile
// classifier and kernel dispatch.  See include/waveprune.h for the contract.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "../../include/waveprune.h"
#include "wp_internal.h"

#include <vector>

namespace {

thread_local char g_last_error[512] = "";

wp_status fail(wp_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

wp_status ok() {
  g_last_error[0] = '\0';
  return WP_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Prefill and decode: groups of 16 or 32 dims (one or two MFMA steps per
// group) and the fine groups 2, 4, 8 (G = 2 is one cutoff per channel, the
// exact rule).  The backward pass and the compact K store take 16 or 32.
bool supported_shape(int32_t d_h, int32_t G) {
  return (d_h == 64 || d_h == 128) && (G == 2 || G == 4 || G == 8 || G == 16 || G == 32);
}

bool supported_coarse(int32_t d_h, int32_t G) {
  return (d_h == 64 || d_h == 128) && (G == 16 || G == 32);
}

// Cutoffs must be a non-decreasing, non-negative table: the tile classes
// then form a skip prefix / partial middle / full suffix.
wp_status check_cutoffs(const int32_t* cut, int32_t ng) {
  for (int g = 0; g < ng; ++g) {
    if (cut[g] < 0) return fail(WP_ERR_ARG, "cutoffs[%d] = %d is negative", g, cut[g]);
    if (g > 0 && cut[g] < cut[g - 1])
      return fail(WP_ERR_ARG, "cutoffs must be non-decreasing (cutoffs[%d] = %d < cutoffs[%d] = %d)",
                  g, cut[g], g - 1, cut[g - 1]);
  }
  return WP_OK;
}

wp_status check_strides(const int64_t* st, int count) {
  for (int i = 0; i < count; ++i) {
    if (st[i] < 0) return fail(WP_ERR_SHAPE, "stride %d is negative (%lld)", i, (long long)st[i]);
    if (st[i] % 8) return fail(WP_ERR_ALIGN, "stride %d = %lld is not a multiple of 8 elements",
                               i, (long long)st[i]);
  }
  return WP_OK;
}

// Rows of K, V (and in the backward Q, dO) are read through 32-bit buffer
// resources that span one tile of `rows` tokens: the tile's byte span, and
// the byte stride itself, must stay below 2^31.
bool tile_span_ok(int64_t token_stride, int32_t d_h, int rows) {
  return token_stride * 2 < 2147483647LL && (int64_t)(rows - 1) * token_stride * 2 + 2 * d_h < 2147483647LL;
}

// Classes of one tile with causal distances [lD, rD]: skip groups
// [0, splitL), partial [splitL, splitR), full [splitR, ng).
inline void add_tile(const int32_t* cut, int ng, int64_t lD, int64_t rD, int64_t* counts) {
  int sL = 0, sR = 0;
  for (int g = 0; g < ng; ++g) {
    sL += cut[g] < lD;
    sR += cut[g] < rD;
  }
  for (int g = 0; g < ng; ++g) counts[3 * g + (g < sL ? 0 : (g < sR ? 1 : 2))] += 1;
  counts[3 * ng] += 1;
}

}  // namespace

extern "C" {

const char* wp_version(void) { return "0.1.0"; }

const char* wp_last_error(void) { return g_last_error; }

const char* wp_status_string(wp_status s) {
  switch (s) {
    case WP_OK: return "ok";
    case WP_ERR_NULL: return "null pointer";
    case WP_ERR_SHAPE: return "bad shape";
    case WP_ERR_UNSUPPORTED: return "unsupported head dim or group size";
    case WP_ERR_ALIGN: return "misaligned pointer or stride";
    case WP_ERR_WORKSPACE: return "workspace too small";
    case WP_ERR_ARG: return "bad argument";
    case WP_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

wp_status wp_group_cutoffs(double theta, int32_t d_h, int32_t G, double pos_scale, int32_t* out,
                           int32_t out_len) {
  if (!out) return fail(WP_ERR_NULL, "out is NULL");
  if (!(theta > 0.0) || !isfinite(theta)) return fail(WP_ERR_ARG, "theta must be finite and > 0");
  if (!(pos_scale > 0.0) || !isfinite(pos_scale))
    return fail(WP_ERR_ARG, "pos_scale must be finite and > 0");
  if (d_h <= 0 || d_h % 2) return fail(WP_ERR_SHAPE, "d_h = %d must be positive and even", d_h);
  if (G <= 0 || G % 2 || d_h % G) return fail(WP_ERR_SHAPE, "G = %d must be even and divide d_h", G);
  if (out_len != d_h / G) return fail(WP_ERR_SHAPE, "out_len = %d, expected d_h/G = %d", out_len, d_h / G);
  const double two_pi = 6.283185307179586476925286766559;
  for (int g = 0; g < out_len; ++g) {
    double best = -1.0;
    // channels of dims [gG, (g+1)G) are c = gG/2 .. (g+1)G/2 - 1
    for (int c = g * G / 2; c < (g + 1) * G / 2; ++c) {
      const double f = pow(theta, -2.0 * (double)c / (double)d_h) / pos_scale;   // scaled frequency
      const double w = floor(two_pi / f);                                        // kept distances
      if (w > best) best = w;
    }
    out[g] = (best >= 2147483647.0 || !isfinite(best)) ? WP_NEVER_PRUNE : (int32_t)best;
  }
  return ok();
}

wp_status wp_cutoffs_from_freqs(const double* freqs, int32_t n_ch, double alpha, int32_t trunc_channels,
                                int32_t G, int32_t* out, int32_t out_len) {
  if (!freqs || !out) return fail(WP_ERR_NULL, "freqs/out is NULL");
  if (n_ch <= 0) return fail(WP_ERR_SHAPE, "n_ch = %d must be positive", n_ch);
  if (trunc_channels < 0 || trunc_channels > n_ch)
    return fail(WP_ERR_SHAPE, "trunc_channels = %d must be in [0, n_ch = %d]", trunc_channels, n_ch);
  if (G <= 0 || G % 2 || (2 * (int64_t)n_ch) % G)
    return fail(WP_ERR_SHAPE, "G = %d must be even and divide d_h = 2*n_ch = %lld", G, 2LL * n_ch);
  if ((int64_t)out_len * G != 2 * (int64_t)n_ch)
    return fail(WP_ERR_SHAPE, "out_len = %d, expected 2*n_ch/G = %lld", out_len, 2LL * n_ch / G);
  if (!(alpha > 0.0)) return fail(WP_ERR_ARG, "alpha must be > 0 (or +infinity)");
  for (int c = 0; c < n_ch; ++c)
    if (!(freqs[c] > 0.0) || !isfinite(freqs[c]))
      return fail(WP_ERR_ARG, "freqs[%d] must be finite and > 0", c);
  const double pi = 3.14159265358979323846264338327950288;
  std::vector<int32_t> tab(out_len);
  for (int g = 0; g < out_len; ++g) {
    double best = -1.0;
    // channels of dims [gG, (g+1)G) are c = gG/2 .. (g+1)G/2 - 1
    for (int c = g * G / 2; c < (g + 1) * G / 2; ++c) {
      // window alpha*pi/f_c; channels from trunc_channels on are never pruned
      const double w = (c < trunc_channels && isfinite(alpha)) ? floor(alpha * pi / freqs[c]) : INFINITY;
      if (w > best) best = w;
    }
    tab[g] = (best >= 2147483647.0 || !isfinite(best)) ? WP_NEVER_PRUNE : (int32_t)best;
  }
  for (int g = 1; g < out_len; ++g)
    if (tab[g] < tab[g - 1])
      return fail(WP_ERR_ARG, "group cutoffs decrease at group %d (%d < %d): the kernels need a "
                              "non-decreasing table (frequencies non-increasing over the groups)",
                  g, tab[g], tab[g - 1]);
  for (int g = 0; g < out_len; ++g) out[g] = tab[g];
  return ok();
}

wp_status wp_prefill_tiling(int32_t d_h, int32_t G, int32_t* BM, int32_t* BN) {
  if (!BM || !BN) return fail(WP_ERR_NULL, "BM/BN is NULL");
  if (!supported_shape(d_h, G)) return fail(WP_ERR_UNSUPPORTED, "d_h=%d G=%d unsupported", d_h, G);
  *BM = wp::kPrefillBM;
  *BN = wp::kPrefillBN;
  return ok();
}

wp_status wp_decode_tiling(int32_t d_h, int32_t G, int32_t* BN) {
  if (!BN) return fail(WP_ERR_NULL, "BN is NULL");
  if (!supported_shape(d_h, G)) return fail(WP_ERR_UNSUPPORTED, "d_h=%d G=%d unsupported", d_h, G);
  *BN = wp::kDecodeBN;
  return ok();
}

wp_status wp_prefill_tile_counts(int32_t n, int32_t d_h, int32_t G, const int32_t* cutoffs,
                                 int64_t* counts) {
  if (!cutoffs || !counts) return fail(WP_ERR_NULL, "cutoffs/counts is NULL");
  if (!supported_shape(d_h, G)) return fail(WP_ERR_UNSUPPORTED, "d_h=%d G=%d unsupported", d_h, G);
  if (n < 1) return fail(WP_ERR_SHAPE, "n = %d must be >= 1", n);
  const int ng = d_h / G;
  if (wp_status s = check_cutoffs(cutoffs, ng)) return s;
  memset(counts, 0, sizeof(int64_t) * (3 * ng + 1));
  const int BM = wp::kPrefillBM, BN = wp::kPrefillBN;
  for (int64_t i0 = 0; i0 < n; i0 += BM) {
    const int64_t i1 = (i0 + BM < n ? i0 + BM : n) - 1;
    for (int64_t j0 = 0; j0 <= i1; j0 += BN) {
      const int64_t j1 = (j0 + BN < n ? j0 + BN : n) - 1;
      const int64_t lD = i0 - j1 > 0 ? i0 - j1 : 0;
      add_tile(cutoffs, ng, lD, i1 - j0, counts);
    }
  }
  return ok();
}

wp_status wp_decode_tile_counts(int32_t q_pos, int32_t cache_len, int32_t d_h, int32_t G,
                                const int32_t* cutoffs, int64_t* counts) {
  if (!cutoffs || !counts) return fail(WP_ERR_NULL, "cutoffs/counts is NULL");
  if (!supported_shape(d_h, G)) return fail(WP_ERR_UNSUPPORTED, "d_h=%d G=%d unsupported", d_h, G);
  if (cache_len < 0) return fail(WP_ERR_SHAPE, "cache_len = %d must be >= 0", cache_len);
  if (cache_len > 0 && q_pos < cache_len - 1)
    return fail(WP_ERR_ARG, "q_pos = %d must be >= cache_len - 1 = %d", q_pos, cache_len - 1);
  const int ng = d_h / G;
  if (wp_status s = check_cutoffs(cutoffs, ng)) return s;
  memset(counts, 0, sizeof(int64_t) * (3 * ng + 1));
  const int BN = wp::kDecodeBN;
  for (int64_t j0 = 0; j0 < cache_len; j0 += BN) {
    const int64_t j1 = (j0 + BN < cache_len ? j0 + BN : cache_len) - 1;
    add_tile(cutoffs, ng, (int64_t)q_pos - j1, (int64_t)q_pos - j0, counts);
  }
  return ok();
}

wp_status wp_rope_apply(const void* x, int32_t x_dtype, void* y, int32_t B, int32_t n, int32_t H,
                        int32_t d_h, const int64_t x_strides[3], const int64_t y_strides[3],
                        const int64_t* pos_start, double theta, double pos_scale, void* stream) {
  if (!x || !y || !x_strides || !y_strides) return fail(WP_ERR_NULL, "x, y or strides is NULL");
  if (x_dtype != WP_DTYPE_BF16 && x_dtype != WP_DTYPE_F32)
    return fail(WP_ERR_ARG, "x_dtype = %d must be WP_DTYPE_BF16 or WP_DTYPE_F32", x_dtype);
  if (d_h != 64 && d_h != 128) return fail(WP_ERR_UNSUPPORTED, "d_h = %d unsupported", d_h);
  if (B < 1 || n < 1 || H < 1) return fail(WP_ERR_SHAPE, "B, n, H must be >= 1");
  if ((int64_t)B * n > 2147483647LL) return fail(WP_ERR_SHAPE, "B*n exceeds 2^31-1");
  if (!(theta > 0.0) || !isfinite(theta)) return fail(WP_ERR_ARG, "theta must be finite and > 0");
  if (!(pos_scale > 0.0) || !isfinite(pos_scale))
    return fail(WP_ERR_ARG, "pos_scale must be finite and > 0");
  if (!aligned16(x) || !aligned16(y)) return fail(WP_ERR_ALIGN, "x and y must be 16-byte aligned");
  if (wp_status s = check_strides(x_strides, 3)) return s;
  if (wp_status s = check_strides(y_strides, 3)) return s;
  if (x == y) {
    if (x_dtype != WP_DTYPE_BF16 || memcmp(x_strides, y_strides, 3 * sizeof(int64_t)) != 0)
      return fail(WP_ERR_ARG, "in-place RoPE needs a bf16 input with identical strides");
  }
  if (pos_start && (reinterpret_cast<uintptr_t>(pos_start) & 7u))
    return fail(WP_ERR_ALIGN, "pos_start must be 8-byte aligned");
  wp::RopeArgs a;
  memset(&a, 0, sizeof(a));
  a.x = x;
  a.y = y;
  a.pos_start = pos_start;
  a.xs_b = x_strides[0]; a.xs_t = x_strides[1]; a.xs_h = x_strides[2];
  a.ys_b = y_strides[0]; a.ys_t = y_strides[1]; a.ys_h = y_strides[2];
  a.B = B; a.n = n; a.H = H; a.d_h = d_h;
  a.x_f32 = (x_dtype == WP_DTYPE_F32);
  for (int c = 0; c < d_h / 2; ++c)
    a.inv_freq[c] = pow(theta, -2.0 * (double)c / (double)d_h) / pos_scale;
  hipError_t e = wp::launch_rope(a, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(WP_ERR_HIP, "rope launch: %s", hipGetErrorString(e));
  return ok();
}

wp_status wp_prefill(const void* q, const void* k, const void* v, void* o, float* lse, int32_t B,
                     int32_t n, int32_t Hq, int32_t Hkv, int32_t d_h, const int64_t strides[12],
                     const int32_t* cutoffs, int32_t G, uint32_t flags, int64_t* counters,
                     void* stream) {
  if (!q || !k || !v || !o || !strides) return fail(WP_ERR_NULL, "q, k, v, o or strides is NULL");
  if (flags & ~(WP_FLAG_DENSE | WP_FLAG_COUNT | WP_FLAG_MFMA16))
    return fail(WP_ERR_ARG, "unknown flags 0x%x", flags);
  const bool dense = flags & WP_FLAG_DENSE;
  const bool count = flags & WP_FLAG_COUNT;
  const bool mfma16 = flags & WP_FLAG_MFMA16;
  if (!dense && !cutoffs) return fail(WP_ERR_NULL, "cutoffs is NULL (and WP_FLAG_DENSE not set)");
  if (count && !counters) return fail(WP_ERR_NULL, "counters is NULL with WP_FLAG_COUNT");
  if (!supported_shape(d_h, G)) return fail(WP_ERR_UNSUPPORTED, "d_h=%d G=%d unsupported", d_h, G);
  if (mfma16 && !(d_h == 128 && G == 32))
    return fail(WP_ERR_UNSUPPORTED, "WP_FLAG_MFMA16 takes d_h = 128 and G = 32 (d_h=%d G=%d)", d_h, G);
  if (B < 1 || n < 1 || Hq < 1 || Hkv < 1) return fail(WP_ERR_SHAPE, "B, n, Hq, Hkv must be >= 1");
  if (Hq % Hkv) return fail(WP_ERR_SHAPE, "Hq = %d is not a multiple of Hkv = %d", Hq, Hkv);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(WP_ERR_ALIGN, "q, k, v, o must be 16-byte aligned");
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return fail(WP_ERR_ALIGN, "lse misaligned");
  if (counters && (reinterpret_cast<uintptr_t>(counters) & 7u))
    return fail(WP_ERR_ALIGN, "counters must be 8-byte aligned");
  if (wp_status s = check_strides(strides, 12)) return s;
  // K/V rows are fetched through buffer resources, one per 64-key tile: rows
  // must not overlap and one tile's rows must span less than 2^31 bytes (any
  // sequence length)
  if (strides[4] < d_h || strides[7] < d_h)
    return fail(WP_ERR_SHAPE, "k/v token strides must be >= d_h");
  if (!tile_span_ok(strides[4], d_h, 64) || !tile_span_ok(strides[7], d_h, 64))
    return fail(WP_ERR_SHAPE, "a 64-token tile of K or V spans 2^31 bytes or more (token stride too large)");
  const int ng = d_h / G;
  wp::PrefillArgs a;
  memset(&a, 0, sizeof(a));
  if (dense) {
    for (int g = 0; g < wp::kMaxGroups; ++g) a.cut[g] = WP_NEVER_PRUNE;
  } else {
    if (wp_status s = check_cutoffs(cutoffs, ng)) return s;
    for (int g = 0; g < ng; ++g) a.cut[g] = cutoffs[g];
  }
  a.q = static_cast<const wp::bf16*>(q);
  a.k = static_cast<const wp::bf16*>(k);
  a.v = static_cast<const wp::bf16*>(v);
  a.o = static_cast<wp::bf16*>(o);
  a.lse = lse;
  a.counters = reinterpret_cast<unsigned long long*>(counters);
  a.qs_b = strides[0]; a.qs_t = strides[1]; a.qs_h = strides[2];
  a.ks_b = strides[3]; a.ks_t = strides[4]; a.ks_h = strides[5];
  a.vs_b = strides[6]; a.vs_t = strides[7]; a.vs_h = strides[8];
  a.os_b = strides[9]; a.os_t = strides[10]; a.os_h = strides[11];
  a.B = B; a.n = n; a.Hq = Hq; a.Hkv = Hkv;
  a.r = Hq / Hkv;
  a.HPW = (a.r % 4 == 0) ? 4 : (a.r % 2 == 0 ? 2 : 1);
  a.HG = a.r / a.HPW;
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)d_h));
  // the query sub-blocks per workgroup (QSUB, QB, nqb) follow from the
  // kernel's wave count and are set by launch_prefill; 32 queries per wave
  // is the smallest workgroup, so this bounds every grid
  const long long max_blocks = (long long)B * Hkv * a.HG * ((n + 31) / 32);
  if (max_blocks > 2147483647LL) return fail(WP_ERR_SHAPE, "grid too large");
  hipError_t e = mfma16 ? wp::launch_prefill16(a, count, reinterpret_cast<hipStream_t>(stream))
                        : wp::launch_prefill(a, d_h, G, count, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(WP_ERR_HIP, "prefill launch: %s", hipGetErrorString(e));
  return ok();
}

namespace {
// compute units of the current device (256 on MI355X; fewer in a partition)
int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    return 256;
  return cus;
}
}  // namespace

int32_t wp_decode_num_splits(int32_t B, int32_t Lmax, int32_t Hkv) {
  if (B < 1 || Hkv < 1 || Lmax < 1) return 1;
  // A decode workgroup fills one CU, and every split of a (sequence, kv
  // head) does the same work, so the kernel takes about
  // ceil(units * S / CUs) rounds of L / S keys: pick the S with the fewest
  // keys per CU (the smallest such S), at least 128 keys per split.
  const long long units = (long long)B * Hkv;
  const long long cus = device_cus();
  long long max_s = ((long long)Lmax + 127) / 128;
  if (max_s > 4 * cus) max_s = 4 * cus;
  long long best = 1;
  double best_cost = (double)((units + cus - 1) / cus);
  for (long long s = 2; s <= max_s; ++s) {
    const double cost = (double)((units * s + cus - 1) / cus) / (double)s;
    if (cost < best_cost * (1.0 - 1e-9)) {
      best = s;
      best_cost = cost;
    }
  }
  return (int32_t)best;
}

namespace {
// number of splits: the requested (or automatic) count, at most one per
// key block of the cache
int decode_splits(int32_t B, int32_t Lmax, int32_t Hkv, int32_t num_splits) {
  long long s = num_splits > 0 ? num_splits : wp_decode_num_splits(B, Lmax, Hkv);
  const long long blocks = ((long long)Lmax + wp::kDecodeBN - 1) / wp::kDecodeBN;
  if (s > blocks) s = blocks;
  return (int)(s < 1 ? 1 : s);
}
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
}  // namespace

size_t wp_decode_workspace_size(int32_t B, int32_t Lmax, int32_t Hq, int32_t Hkv, int32_t d_h,
                                int32_t num_splits) {
  if (B < 1 || Lmax < 1 || Hq < 1 || Hkv < 1 || d_h < 1) return 0;
  const int S = decode_splits(B, Lmax, Hkv, num_splits);
  const size_t rows = (size_t)B * Hq * S;
  return align256(rows * d_h * sizeof(float)) + align256(rows * 2 * sizeof(float));
}

namespace {
// ring sizes and element offsets of the compact K store of one (sequence,
// kv head): group g keeps the last min(Lmax, cutoffs[g] + 1) keys
void kcache_geometry(int32_t Lmax, int32_t ng, int32_t G, const int32_t* cut, int* cap, int64_t* off) {
  off[0] = 0;
  for (int g = 0; g < ng; ++g) {
    const int64_t c = (int64_t)cut[g] + 1;
    cap[g] = (int)(c < Lmax ? c : Lmax);
    off[g + 1] = off[g] + (int64_t)cap[g] * G;
  }
}

// shared by wp_decode and wp_decode_kcache; st10 = {q_b, q_h, k_b, k_t, k_h,
// v_b, v_t, v_h, o_b, o_h} (for the compact store k_b, k_h are its sequence
// and kv-head strides and k_t is unused)
wp_status decode_impl(const void* q, const void* k, const void* v_cache, void* o, const int32_t* cache_len,
                      const int32_t* q_pos, int32_t B, int32_t Lmax, int32_t Hq, int32_t Hkv, int32_t d_h,
                      const int64_t st10[10], const int32_t* cutoffs, int32_t G, int32_t num_splits,
                      void* workspace, size_t workspace_bytes, uint32_t flags, int64_t* counters,
                      void* stream, bool compact) {
  if (flags & ~(WP_FLAG_DENSE | WP_FLAG_COUNT)) return fail(WP_ERR_ARG, "unknown flags 0x%x", flags);
  const bool dense = flags & WP_FLAG_DENSE;
  const bool count = flags & WP_FLAG_COUNT;
  if (compact && dense) return fail(WP_ERR_ARG, "WP_FLAG_DENSE does not apply to the compact K store");
  if (!dense && !cutoffs) return fail(WP_ERR_NULL, "cutoffs is NULL (and WP_FLAG_DENSE not set)");
  if (count && !counters) return fail(WP_ERR_NULL, "counters is NULL with WP_FLAG_COUNT");
  if (!supported_shape(d_h, G)) return fail(WP_ERR_UNSUPPORTED, "d_h=%d G=%d unsupported", d_h, G);
  if (compact && !supported_coarse(d_h, G))
    return fail(WP_ERR_UNSUPPORTED, "the compact K store takes G = 16 or 32 (G=%d)", G);
  if (B < 1 || Lmax < 1 || Hq < 1 || Hkv < 1) return fail(WP_ERR_SHAPE, "B, Lmax, Hq, Hkv must be >= 1");
  if (Hq % Hkv) return fail(WP_ERR_SHAPE, "Hq = %d is not a multiple of Hkv = %d", Hq, Hkv);
  if (num_splits < 0) return fail(WP_ERR_ARG, "num_splits must be >= 0");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v_cache) || !aligned16(o))
    return fail(WP_ERR_ALIGN, "q, the K cache or store, v_cache, o must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(workspace) & 255u)
    return fail(WP_ERR_ALIGN, "workspace must be 256-byte aligned");
  if ((reinterpret_cast<uintptr_t>(cache_len) & 3u) || (reinterpret_cast<uintptr_t>(q_pos) & 3u))
    return fail(WP_ERR_ALIGN, "cache_len / q_pos misaligned");
  if (counters && (reinterpret_cast<uintptr_t>(counters) & 7u))
    return fail(WP_ERR_ALIGN, "counters must be 8-byte aligned");
  if (wp_status s = check_strides(st10, 10)) return s;
  if ((!compact && st10[3] < d_h) || st10[6] < d_h)
    return fail(WP_ERR_SHAPE, "k/v cache token strides must be >= d_h");
  if ((!compact && !tile_span_ok(st10[3], d_h, 32)) || !tile_span_ok(st10[6], d_h, 32))
    return fail(WP_ERR_SHAPE, "a 32-token block of the K or V cache spans 2^31 bytes or more (token stride too large)");
  const size_t need = wp_decode_workspace_size(B, Lmax, Hq, Hkv, d_h, num_splits);
  if (workspace_bytes < need)
    return fail(WP_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, need);
  const int ng = d_h / G;
  wp::DecodeArgs a;
  memset(&a, 0, sizeof(a));
  if (dense) {
    for (int g = 0; g < wp::kMaxGroups; ++g) a.cut[g] = WP_NEVER_PRUNE;
  } else {
    if (wp_status s = check_cutoffs(cutoffs, ng)) return s;
    for (int g = 0; g < ng; ++g) a.cut[g] = cutoffs[g];
  }
  if (compact) {
    if (Lmax > (1 << 24)) return fail(WP_ERR_SHAPE, "the compact K store supports Lmax <= 2^24");
    int64_t off[wp::kMaxCacheGroups + 1];
    kcache_geometry(Lmax, ng, G, cutoffs, a.kcap, off);
    if (st10[2] < off[ng] || st10[4] < off[ng])
      return fail(WP_ERR_SHAPE, "K store strides must be >= the store size (%lld elements)", (long long)off[ng]);
    if (off[ng] * 2 >= 2147483647LL) return fail(WP_ERR_SHAPE, "one K store spans 2^31 bytes or more");
    for (int g = 0; g < ng; ++g) a.koff[g] = (int)off[g];
    a.kstore_elems = (int)off[ng];
    a.compact = 1;
  }
  const int S = decode_splits(B, Lmax, Hkv, num_splits);
  const size_t rows = (size_t)B * Hq * S;
  a.q = static_cast<const wp::bf16*>(q);
  a.k = static_cast<const wp::bf16*>(k);
  a.v = static_cast<const wp::bf16*>(v_cache);
  a.o = static_cast<wp::bf16*>(o);
  a.cache_len = cache_len;
  a.q_pos = q_pos;
  a.part_o = static_cast<float*>(workspace);
  a.part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + align256(rows * d_h * sizeof(float)));
  a.counters = reinterpret_cast<unsigned long long*>(counters);
  a.qs_b = st10[0]; a.qs_h = st10[1];
  a.ks_b = st10[2]; a.ks_t = st10[3]; a.ks_h = st10[4];
  a.vs_b = st10[5]; a.vs_t = st10[6]; a.vs_h = st10[7];
  a.os_b = st10[8]; a.os_h = st10[9];
  a.B = B; a.Lmax = Lmax; a.Hkv = Hkv;
  a.rs = Hq / Hkv;
  a.S = S;
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)d_h));
  const long long blocks = (long long)B * Hkv * S;
  if (blocks > 2147483647LL || (long long)B * Hq > 2147483647LL)
    return fail(WP_ERR_SHAPE, "grid too large");
  // The kernel holds at most 32 query heads of a kv head as MFMA columns
  // (two sets of 16 sharing each K / V operand).  More heads per kv head run
  // in passes of 32 (each pass reads the cache again; tile counts are taken
  // in the first pass only); the passes share the workspace in stream order.
  for (int h0 = 0; h0 < a.rs; h0 += 32) {
    wp::DecodeArgs p = a;
    p.r = a.rs - h0 < 32 ? a.rs - h0 : 32;
    p.Hq = Hkv * p.r;
    p.q = a.q + (int64_t)h0 * a.qs_h;
    p.o = a.o + (int64_t)h0 * a.os_h;
    hipError_t e = wp::launch_decode(p, d_h, G, count && h0 == 0, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(WP_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
  }
  return ok();
}
}  // namespace

wp_status wp_decode(const void* q, const void* k_cache, const void* v_cache, void* o,
                    const int32_t* cache_len, const int32_t* q_pos, int32_t B, int32_t Lmax,
                    int32_t Hq, int32_t Hkv, int32_t d_h, const int64_t strides[10],
                    const int32_t* cutoffs, int32_t G, int32_t num_splits, void* workspace,
                    size_t workspace_bytes, uint32_t flags, int64_t* counters, void* stream) {
  if (!q || !k_cache || !v_cache || !o || !cache_len || !q_pos || !strides || !workspace)
    return fail(WP_ERR_NULL, "a required pointer is NULL");
  return decode_impl(q, k_cache, v_cache, o, cache_len, q_pos, B, Lmax, Hq, Hkv, d_h, strides, cutoffs, G,
                     num_splits, workspace, workspace_bytes, flags, counters, stream, false);
}

wp_status wp_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, void* o,
                            const int32_t* cache_len, const int32_t* q_pos, int32_t B, int32_t Lmax,
                            int32_t Hq, int32_t Hkv, int32_t d_h, const int64_t strides[10],
                            const int32_t* cutoffs, int32_t G, int32_t num_splits, uint32_t flags,
                            int64_t* counters, void* stream) {
  if (!q || !k_cache || !v_cache || !o || !cache_len || !q_pos || !strides)
    return fail(WP_ERR_NULL, "a required pointer is NULL");
  if (B < 1 || Lmax < 1 || Hq < 1 || Hkv < 1 || d_h < 1)
    return fail(WP_ERR_SHAPE, "B, Lmax, Hq, Hkv, d_h must be >= 1");
  if (num_splits < 0) return fail(WP_ERR_ARG, "num_splits must be >= 0");
  const size_t need = wp_decode_workspace_size(B, Lmax, Hq, Hkv, d_h, num_splits);
  if (need > wp::kDecodeScratchBytes)
    return fail(WP_ERR_WORKSPACE,
                "the partial results need %zu bytes, more than the %zu-byte device scratch of "
                "wp_decode_noalloc (use wp_decode with a workspace, or fewer splits)",
                need, wp::kDecodeScratchBytes);
  void* scratch = nullptr;
  hipError_t e = wp::decode_scratch(&scratch);
  if (e != hipSuccess) return fail(WP_ERR_HIP, "decode scratch address: %s", hipGetErrorString(e));
  return decode_impl(q, k_cache, v_cache, o, cache_len, q_pos, B, Lmax, Hq, Hkv, d_h, strides, cutoffs, G,
                     num_splits, scratch, wp::kDecodeScratchBytes, flags, counters, stream, false);
}

size_t wp_prefill_backward_workspace_size(int32_t B, int32_t n, int32_t Hq) {
  if (B < 1 || n < 1 || Hq < 1) return 0;
  return align256((size_t)B * Hq * n * 2 * sizeof(float));
}

wp_status wp_prefill_backward(const void* q, const void* k, const void* v, const void* o, const void* dout,
                              const float* lse, void* dq, void* dk, void* dv, int32_t B, int32_t n,
                              int32_t Hq, int32_t Hkv, int32_t d_h, const int64_t strides[24],
                              const int32_t* cutoffs, int32_t G, uint32_t flags, void* workspace,
                              size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !strides || !workspace)
    return fail(WP_ERR_NULL, "a required pointer is NULL");
  if (flags & ~WP_FLAG_DENSE) return fail(WP_ERR_ARG, "unknown flags 0x%x", flags);
  const bool dense = flags & WP_FLAG_DENSE;
  if (!dense && !cutoffs) return fail(WP_ERR_NULL, "cutoffs is NULL (and WP_FLAG_DENSE not set)");
  if (!supported_shape(d_h, G)) return fail(WP_ERR_UNSUPPORTED, "d_h=%d G=%d unsupported", d_h, G);
  if (B < 1 || n < 1 || Hq < 1 || Hkv < 1) return fail(WP_ERR_SHAPE, "B, n, Hq, Hkv must be >= 1");
  if (Hq % Hkv) return fail(WP_ERR_SHAPE, "Hq = %d is not a multiple of Hkv = %d", Hq, Hkv);
  const void* ptrs[8] = {q, k, v, o, dout, dq, dk, dv};
  for (const void* p : ptrs)
    if (!aligned16(p)) return fail(WP_ERR_ALIGN, "q, k, v, o, dO, dQ, dK, dV must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(lse) & 3u) return fail(WP_ERR_ALIGN, "lse misaligned");
  if (reinterpret_cast<uintptr_t>(workspace) & 255u)
    return fail(WP_ERR_ALIGN, "workspace must be 256-byte aligned");
  if (wp_status s = check_strides(strides, 24)) return s;
  // Q, dO (dK/dV kernel) and K, V (dQ kernel) rows are fetched through
  // buffer resources: token strides >= d_h, one 64-token tile < 2^31 bytes
  const int tok[4] = {1, 4, 7, 13};
  for (int t : tok) {
    if (strides[t] < d_h) return fail(WP_ERR_SHAPE, "q, k, v, dO token strides must be >= d_h");
    if (!tile_span_ok(strides[t], d_h, 64))
      return fail(WP_ERR_SHAPE, "a 64-token tile of q, k, v or dO spans 2^31 bytes or more (token stride too large)");
  }
  const size_t need = wp_prefill_backward_workspace_size(B, n, Hq);
  if (workspace_bytes < need)
    return fail(WP_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, need);
  const int ng = d_h / G;
  wp::BackwardArgs a;
  memset(&a, 0, sizeof(a));
  if (dense) {
    for (int g = 0; g < wp::kMaxGroups; ++g) a.cut[g] = WP_NEVER_PRUNE;
  } else {
    if (wp_status s = check_cutoffs(cutoffs, ng)) return s;
    for (int g = 0; g < ng; ++g) a.cut[g] = cutoffs[g];
  }
  a.q = static_cast<const wp::bf16*>(q);
  a.k = static_cast<const wp::bf16*>(k);
  a.v = static_cast<const wp::bf16*>(v);
  a.o = static_cast<const wp::bf16*>(o);
  a.dout = static_cast<const wp::bf16*>(dout);
  a.lse = lse;
  a.rowv = static_cast<float*>(workspace);
  a.dq = static_cast<wp::bf16*>(dq);
  a.dk = static_cast<wp::bf16*>(dk);
  a.dv = static_cast<wp::bf16*>(dv);
  int64_t* st[8][3] = {{&a.qs_b, &a.qs_t, &a.qs_h},    {&a.ks_b, &a.ks_t, &a.ks_h},
                       {&a.vs_b, &a.vs_t, &a.vs_h},    {&a.os_b, &a.os_t, &a.os_h},
                       {&a.gs_b, &a.gs_t, &a.gs_h},    {&a.dqs_b, &a.dqs_t, &a.dqs_h},
                       {&a.dks_b, &a.dks_t, &a.dks_h}, {&a.dvs_b, &a.dvs_t, &a.dvs_h}};
  for (int t = 0; t < 8; ++t)
    for (int c = 0; c < 3; ++c) *st[t][c] = strides[3 * t + c];
  a.B = B; a.n = n; a.Hq = Hq; a.Hkv = Hkv;
  a.r = Hq / Hkv;
  a.HPW = (a.r % 4 == 0) ? 4 : (a.r % 2 == 0 ? 2 : 1);
  a.HG = a.r / a.HPW;
  a.scale = (float)(1.0 / sqrt((double)d_h));
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)d_h));
  if ((long long)B * Hkv * ((n + 31) / 32) * a.HG > 2147483647LL ||
      (long long)B * n * Hq / 256 + 1 > 2147483647LL)
    return fail(WP_ERR_SHAPE, "grid too large");
  hipError_t e = wp::launch_backward(a, d_h, G, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(WP_ERR_HIP, "backward launch: %s", hipGetErrorString(e));
  return ok();
}

wp_status wp_kcache_layout(int32_t Lmax, int32_t d_h, int32_t G, const int32_t* cutoffs, int32_t* caps,
                           int64_t* offsets) {
  if (!cutoffs || !caps || !offsets) return fail(WP_ERR_NULL, "cutoffs/caps/offsets is NULL");
  if (!supported_coarse(d_h, G)) return fail(WP_ERR_UNSUPPORTED, "d_h=%d G=%d unsupported", d_h, G);
  if (Lmax < 1) return fail(WP_ERR_SHAPE, "Lmax must be >= 1");
  const int ng = d_h / G;
  if (wp_status s = check_cutoffs(cutoffs, ng)) return s;
  int cap[wp::kMaxCacheGroups];
  int64_t off[wp::kMaxCacheGroups + 1];
  kcache_geometry(Lmax, ng, G, cutoffs, cap, off);
  for (int g = 0; g < ng; ++g) caps[g] = cap[g];
  for (int g = 0; g <= ng; ++g) offsets[g] = off[g];
  return ok();
}

wp_status wp_kcache_append(const void* k, int32_t B, int32_t T, int32_t Hkv, int32_t d_h,
                           const int64_t k_strides[3], const int32_t* pos0, void* store,
                           const int64_t store_strides[2], int32_t Lmax, const int32_t* cutoffs, int32_t G,
                           void* stream) {
  if (!k || !k_strides || !pos0 || !store || !store_strides || !cutoffs)
    return fail(WP_ERR_NULL, "a required pointer is NULL");
  if (!supported_coarse(d_h, G)) return fail(WP_ERR_UNSUPPORTED, "d_h=%d G=%d unsupported", d_h, G);
  if (B < 1 || T < 1 || Hkv < 1 || Lmax < 1) return fail(WP_ERR_SHAPE, "B, T, Hkv, Lmax must be >= 1");
  if (T > Lmax) return fail(WP_ERR_SHAPE, "T = %d exceeds Lmax = %d", T, Lmax);
  if (Lmax > (1 << 24)) return fail(WP_ERR_SHAPE, "the compact K store supports Lmax <= 2^24");
  if (!aligned16(k) || !aligned16(store)) return fail(WP_ERR_ALIGN, "k and store must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(pos0) & 3u) return fail(WP_ERR_ALIGN, "pos0 misaligned");
  if (wp_status s = check_strides(k_strides, 3)) return s;
  if (wp_status s = check_strides(store_strides, 2)) return s;
  const int ng = d_h / G;
  if (wp_status s = check_cutoffs(cutoffs, ng)) return s;
  wp::KAppendArgs a;
  memset(&a, 0, sizeof(a));
  int64_t off[wp::kMaxCacheGroups + 1];
  kcache_geometry(Lmax, ng, G, cutoffs, a.kcap, off);
  if (store_strides[0] < off[ng] || store_strides[1] < off[ng])
    return fail(WP_ERR_SHAPE, "store strides must be >= the store size (%lld elements)", (long long)off[ng]);
  if (off[ng] * 2 >= 2147483647LL) return fail(WP_ERR_SHAPE, "one K store spans 2^31 bytes or more");
  for (int g = 0; g < ng; ++g) a.koff[g] = (int)off[g];
  a.k = static_cast<const wp::bf16*>(k);
  a.store = static_cast<wp::bf16*>(store);
  a.pos0 = pos0;
  a.ks_b = k_strides[0]; a.ks_t = k_strides[1]; a.ks_h = k_strides[2];
  a.ss_b = store_strides[0]; a.ss_h = store_strides[1];
  a.B = B; a.T = T; a.Hkv = Hkv; a.d_h = d_h; a.G = G; a.ng = ng;
  if ((long long)B * T * Hkv * (d_h / 8) / 256 + 1 > 2147483647LL) return fail(WP_ERR_SHAPE, "grid too large");
  hipError_t e = wp::launch_kcache_append(a, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(WP_ERR_HIP, "kcache append launch: %s", hipGetErrorString(e));
  return ok();
}

wp_status wp_decode_kcache(const void* q, const void* k_store, const void* v_cache, void* o,
                           const int32_t* cache_len, const int32_t* q_pos, int32_t B, int32_t Lmax,
                           int32_t Hq, int32_t Hkv, int32_t d_h, const int64_t strides[9],
                           const int32_t* cutoffs, int32_t G, int32_t num_splits, void* workspace,
                           size_t workspace_bytes, uint32_t flags, int64_t* counters, void* stream) {
  if (!q || !k_store || !v_cache || !o || !cache_len || !q_pos || !strides || !workspace || !cutoffs)
    return fail(WP_ERR_NULL, "a required pointer is NULL");
  const int64_t st10[10] = {strides[0], strides[1], strides[2], 0, strides[3],
                            strides[4], strides[5], strides[6], strides[7], strides[8]};
  return decode_impl(q, k_store, v_cache, o, cache_len, q_pos, B, Lmax, Hq, Hkv, d_h, st10, cutoffs, G,
                     num_splits, workspace, workspace_bytes, flags, counters, stream, true);
}

}  // extern "C"
