// Internal declarations shared by the libwaveprune sources (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wp {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kMaxGroups = 64;      // d_h / G for d_h <= 128, G >= 2 (G = 2: one group per channel)
constexpr int kMaxCacheGroups = 8;  // groups of the compact K store (G >= 16)
constexpr int kMaxChannels = 64;    // d_h / 2 for d_h <= 128

// Tile geometry shared by the kernels, the host classifier and the tiling
// queries.  Prefill: a tile is 32 queries of one head x 64 keys (two 32x32
// MFMA output blocks that share one class per group); decode: a key block of
// 32 keys.
constexpr int kPrefillBM = 32;
constexpr int kPrefillBN = 64;
constexpr int kDecodeBN = 32;

struct RopeArgs {
  const void* x;
  void* y;
  const int64_t* pos_start;
  int64_t xs_b, xs_t, xs_h;
  int64_t ys_b, ys_t, ys_h;
  int B, n, H, d_h;
  int x_f32;
  int rows_per_block;
  double inv_freq[kMaxChannels];   // theta^(-2c/d_h) / pos_scale, float64
};

struct PrefillArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  bf16* o;
  float* lse;
  unsigned long long* counters;
  int64_t qs_b, qs_t, qs_h;
  int64_t ks_b, ks_t, ks_h;
  int64_t vs_b, vs_t, vs_h;
  int64_t os_b, os_t, os_h;
  int B, n, Hq, Hkv;
  int r;        // Hq / Hkv
  int HPW;      // query heads per workgroup
  int QSUB;     // 32-query sub-blocks per workgroup (waves / HPW; set by launch_prefill)
  int HG;       // head groups per kv head (r / HPW)
  int QB;       // queries per workgroup (32 * QSUB; set by launch_prefill)
  int nqb;      // query blocks of QB (set by launch_prefill)
  float scale_log2;   // log2(e) / sqrt(d_h)
  int cut[kMaxGroups];
};

struct DecodeArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  bf16* o;
  const int* cache_len;
  const int* q_pos;
  float* part_o;     // [B][Hq][S][d_h]
  float* part_ml;    // [B][Hq][S][2]
  unsigned long long* counters;
  int64_t qs_b, qs_h;
  int64_t ks_b, ks_t, ks_h;
  int64_t vs_b, vs_t, vs_h;
  int64_t os_b, os_h;
  int B, Lmax, Hq, Hkv;
  int r;          // query heads of each kv head in this launch (<= 32)
  int rs;         // query-head index stride between kv heads (the model's Hq / Hkv)
  int S;          // splits; split s takes key blocks s, s + S, s + 2S, ...
  float scale_log2;
  int cut[kMaxGroups];
  // group-major compact K store (compact != 0): k points at the store and
  // ks_b / ks_h are its sequence / kv-head strides.  The store of one
  // (sequence, kv head) is a ring per group: group g has kcap[g] key slots
  // of G elements at element offset koff[g], and key j sits in slot
  // j % kcap[g], so consecutive keys of a group are contiguous.
  int compact;
  int kstore_elems;   // elements of one (sequence, kv head) store
  int kcap[kMaxCacheGroups];
  int koff[kMaxCacheGroups];
};

// Appending keys to the compact K store: token t of row b (position
// pos0[b] + t) goes, for every group g, to slot (pos0[b] + t) % kcap[g] --
// unless a later token of the same call takes that slot.
struct KAppendArgs {
  const bf16* k;
  bf16* store;
  const int* pos0;
  int64_t ks_b, ks_t, ks_h;
  int64_t ss_b, ss_h;
  int B, T, Hkv, d_h, G, ng;
  int kcap[kMaxCacheGroups];
  int koff[kMaxCacheGroups];
};

// Backward pass of prefill (gradients of <dO, O>).
struct BackwardArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const bf16* o;
  const bf16* dout;
  const float* lse;    // [B][Hq][n], natural log, from the forward pass
  float* rowv;         // [B][Hq][n][2] workspace: (LSE * log2(e), rowsum(dO * O))
  bf16* dq;
  bf16* dk;
  bf16* dv;
  int64_t qs_b, qs_t, qs_h;
  int64_t ks_b, ks_t, ks_h;
  int64_t vs_b, vs_t, vs_h;
  int64_t os_b, os_t, os_h;
  int64_t gs_b, gs_t, gs_h;      // dO
  int64_t dqs_b, dqs_t, dqs_h;
  int64_t dks_b, dks_t, dks_h;
  int64_t dvs_b, dvs_t, dvs_h;
  int B, n, Hq, Hkv;
  int r;          // Hq / Hkv
  int HPW, HG;    // dQ kernel: query heads per workgroup, head groups per kv head
  float scale;        // 1 / sqrt(d_h)
  float scale_log2;   // log2(e) / sqrt(d_h)
  int cut[kMaxGroups];
};

hipError_t launch_rope(const RopeArgs& a, hipStream_t s);
hipError_t launch_prefill(const PrefillArgs& a, int d_h, int G, bool count, hipStream_t s);
// the v_mfma_f32_16x16x32_bf16 prefill (d_h = 128, G = 32)
hipError_t launch_prefill16(const PrefillArgs& a, bool count, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, int d_h, int G, bool count, hipStream_t s);
hipError_t launch_kcache_append(const KAppendArgs& a, hipStream_t s);

// Size of the decode scratch array of each GPU (the allocation-free decode
// entry point keeps its partial results there), and its device address on
// the current device, looked up once per device.
constexpr size_t kDecodeScratchBytes = size_t(8) << 20;   // WP_DECODE_SCRATCH_BYTES
hipError_t decode_scratch(void** ptr);
hipError_t launch_backward(const BackwardArgs& a, int d_h, int G, hipStream_t s);

}  // namespace wp
