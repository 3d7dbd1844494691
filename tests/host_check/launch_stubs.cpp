// Host-side stand-ins for the kernel launchers of libwaveprune, for the
// sanitizer build of the C ABI (api.hip built with AddressSanitizer and
// UndefinedBehaviorSanitizer, run on the CPU).  Instead of launching, each
// stand-in walks the launch's work units with the argument block the kernel
// would receive and touches, through the (host) pointers the caller passed,
// the first and the last byte of every range the kernel addresses: its rows
// of each tensor, every buffer-resource window, the workspace and counters.
// AddressSanitizer then reports any range that leaves its allocation.  The
// test harness passes host memory where the ABI expects device memory; no
// HIP kernel and no device are involved.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../../rope_positional_encoding_amd/csrc/wp_internal.h"

namespace {

volatile unsigned char g_sink;
long long g_touched = 0;

void touch(const void* base, int64_t first_byte, int64_t last_byte) {
  if (last_byte < first_byte) return;
  const unsigned char* p = static_cast<const unsigned char*>(base);
  g_sink = p[first_byte];
  g_sink = p[last_byte];
  g_touched += 2;
}

// bytes [off, off + len) of a bf16 tensor given in elements
void touch_elems(const void* base, int64_t off_elems, int64_t len_elems, int esize = 2) {
  touch(base, off_elems * esize, (off_elems + len_elems) * esize - 1);
}

alignas(256) unsigned char g_scratch[wp::kDecodeScratchBytes];

}  // namespace

extern "C" long long wp_host_check_touched() { return g_touched; }

namespace wp {

hipError_t launch_rope(const RopeArgs& a, hipStream_t) {
  for (int b = 0; b < a.B; ++b)
    for (int t : {0, a.n - 1})
      for (int h : {0, a.H - 1}) {
        touch_elems(a.x, b * a.xs_b + t * a.xs_t + h * a.xs_h, a.d_h, a.x_f32 ? 4 : 2);
        touch_elems(a.y, b * a.ys_b + t * a.ys_t + h * a.ys_h, a.d_h);
      }
  if (a.pos_start) touch(a.pos_start, 0, 8 * a.B - 1);
  return hipSuccess;
}

hipError_t launch_prefill(const PrefillArgs& a, int d_h, int G, bool count, hipStream_t) {
  for (int b = 0; b < a.B; ++b) {
    for (int h = 0; h < a.Hq; ++h)
      for (int i : {0, a.n - 1}) {
        touch_elems(a.q, b * a.qs_b + (int64_t)i * a.qs_t + h * a.qs_h, d_h);
        touch_elems(a.o, b * a.os_b + (int64_t)i * a.os_t + h * a.os_h, d_h);
        if (a.lse) touch_elems(a.lse, ((int64_t)b * a.Hq + h) * a.n + i, 1, 4);
      }
    // K/V buffer windows: from the tile's first key to the sequence end
    for (int kvh = 0; kvh < a.Hkv; ++kvh) {
      touch_elems(a.k, b * a.ks_b + kvh * a.ks_h, (int64_t)(a.n - 1) * a.ks_t + d_h);
      touch_elems(a.v, b * a.vs_b + kvh * a.vs_h, (int64_t)(a.n - 1) * a.vs_t + d_h);
    }
  }
  if (a.r != a.Hq / a.Hkv || a.HPW * a.HG != a.r) return hipErrorInvalidValue;
  if (count) touch_elems(a.counters, 0, 3 * (d_h / G) + 1, 8);
  return hipSuccess;
}

hipError_t launch_prefill16(const PrefillArgs& a, bool count, hipStream_t s) {
  return launch_prefill(a, 128, 32, count, s);
}

hipError_t launch_decode(const DecodeArgs& a, int d_h, int G, bool count, hipStream_t) {
  if (a.r < 1 || a.r > 32 || a.S < 1) return hipErrorInvalidValue;
  for (int b = 0; b < a.B; ++b) {
    touch(a.cache_len, 4 * b, 4 * b + 3);
    touch(a.q_pos, 4 * b, 4 * b + 3);
    const int L = a.cache_len[b] < a.Lmax ? a.cache_len[b] : a.Lmax;
    for (int kvh = 0; kvh < a.Hkv; ++kvh) {
      for (int hh = 0; hh < a.r; ++hh) {
        const int h = kvh * a.rs + hh;   // the head among the model's heads
        touch_elems(a.q, b * a.qs_b + h * a.qs_h, d_h);
        touch_elems(a.o, b * a.os_b + h * a.os_h, d_h);
      }
      if (a.compact)
        touch_elems(a.k, b * a.ks_b + kvh * a.ks_h, a.kstore_elems);
      else if (L > 0)
        touch_elems(a.k, b * a.ks_b + kvh * a.ks_h, (int64_t)(L - 1) * a.ks_t + d_h);
      if (L > 0) touch_elems(a.v, b * a.vs_b + kvh * a.vs_h, (int64_t)(L - 1) * a.vs_t + d_h);
    }
  }
  // partial results [B][Hq][S][d_h] and [B][Hq][S][2] of this launch
  const int64_t rows = (int64_t)a.B * a.Hq * a.S;
  touch_elems(a.part_o, 0, rows * d_h, 4);
  touch_elems(a.part_ml, 0, rows * 2, 4);
  if (count) touch_elems(a.counters, 0, 3 * (d_h / G) + 1, 8);
  return hipSuccess;
}

hipError_t launch_kcache_append(const KAppendArgs& a, hipStream_t) {
  for (int b = 0; b < a.B; ++b) {
    touch(a.pos0, 4 * b, 4 * b + 3);
    for (int h = 0; h < a.Hkv; ++h) {
      for (int t : {0, a.T - 1}) touch_elems(a.k, b * a.ks_b + (int64_t)t * a.ks_t + h * a.ks_h, a.d_h);
      for (int g = 0; g < a.ng; ++g)
        touch_elems(a.store, b * a.ss_b + h * a.ss_h + a.koff[g], (int64_t)a.kcap[g] * a.G);
    }
  }
  return hipSuccess;
}

hipError_t launch_backward(const BackwardArgs& a, int d_h, int, hipStream_t) {
  for (int b = 0; b < a.B; ++b) {
    for (int h = 0; h < a.Hq; ++h)
      for (int i : {0, a.n - 1}) {
        touch_elems(a.q, b * a.qs_b + (int64_t)i * a.qs_t + h * a.qs_h, d_h);
        touch_elems(a.o, b * a.os_b + (int64_t)i * a.os_t + h * a.os_h, d_h);
        touch_elems(a.dout, b * a.gs_b + (int64_t)i * a.gs_t + h * a.gs_h, d_h);
        touch_elems(a.dq, b * a.dqs_b + (int64_t)i * a.dqs_t + h * a.dqs_h, d_h);
        touch_elems(a.lse, ((int64_t)b * a.Hq + h) * a.n + i, 1, 4);
        touch_elems(a.rowv, (((int64_t)b * a.Hq + h) * a.n + i) * 2, 2, 4);
      }
    for (int kvh = 0; kvh < a.Hkv; ++kvh) {
      touch_elems(a.k, b * a.ks_b + kvh * a.ks_h, (int64_t)(a.n - 1) * a.ks_t + d_h);
      touch_elems(a.v, b * a.vs_b + kvh * a.vs_h, (int64_t)(a.n - 1) * a.vs_t + d_h);
      for (int i : {0, a.n - 1}) {
        touch_elems(a.dk, b * a.dks_b + (int64_t)i * a.dks_t + kvh * a.dks_h, d_h);
        touch_elems(a.dv, b * a.dvs_b + (int64_t)i * a.dvs_t + kvh * a.dvs_h, d_h);
      }
    }
  }
  return hipSuccess;
}

hipError_t decode_scratch(void** ptr) {
  *ptr = g_scratch;
  return hipSuccess;
}

}  // namespace wp
