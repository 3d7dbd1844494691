// WavePrune causal prefill attention for gfx950 (grouped rule).
//
// Method: every RoPE channel adds to the QK logit only while the distance is
// within its cutoff; pruned terms are 0 and the key stays in the softmax
// (WavePrune reading notes on cc.laoqi.cc, section 2.1, Eq. (6)).  Head dims
// are grouped (G = 16 or 32) and a group uses the largest cutoff inside it
// (section 2.3, Eq. (8)).  Each (32-query x 64-key) tile is classified per
// group from its distance range [l_D, r_D]: skip, partial or full
// (section 2.3 table).  Because the cutoffs are non-decreasing two split
// points describe a tile: groups [0, splitL) skip, [splitL, splitR) partial,
// [splitR, ng) full (section 2.3, the paragraph on splitL/splitR).
//
// gfx950 design (not the pages' A100 design):
//  * The logits are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: one MFMA contracts exactly 16 head dims, so a
//    G = 16 group is one MFMA per 32x32 block and G = 32 is two.  In S^T the
//    lane owns one query column, so row max / row sum need one cross-half
//    exchange only, and the probabilities are already laid out as the B
//    operand of O^T = V^T P^T.
//  * Skipped groups issue no MFMA; the full groups run as one MFMA chain
//    from the highest group down, leaving the chain with one wave-uniform
//    scalar branch at splitR (the "suffix" GEMM); a partial group gets its
//    own accumulator, is masked with dist <= cutoff, then added, on a
//    separate path that only boundary tiles take.  No per-(splitL, splitR)
//    code specialization is needed.
//  * A workgroup is 4 waves that share one kv head and one key range: with
//    GQA ratio >= 4 the waves are 4 query heads over the same 32 queries
//    (identical tile classes, K/V staged once in LDS for all four).
//  * K is staged row-major in LDS (row pad 16 B: conflict-free 16-byte MFMA
//    operand reads); V is written transposed (V^T) with a key permutation
//    that matches the S^T register layout, so both MFMA operands of P.V are
//    single 16-byte LDS reads.  LDS holds two stages: while tile t is
//    consumed, tile t+1 is written into the other stage and tile t+2 is in
//    flight from HBM into registers; one barrier per tile.
//  * The running max is refreshed (and O rescaled) only when it grows by more
//    than 8 in log2 units, so every probability stays below 2^8; the final
//    O / l and the LSE are unaffected.
//  * Workgroups run heaviest (last query blocks) first; kv head is the
//    fastest-varying block index so that on 8 kv heads each XCD (blocks are
//    dealt round-robin to the 8 XCDs) keeps one kv head's K/V in its L2.
#include "wp_internal.h"

namespace wp {

namespace {

constexpr int kThreads = 256;
// dword 3 of a raw (untyped, stride 0) buffer resource on gfx9-family parts
constexpr int kBufferFlags = 0x00020000;
constexpr int kTileKeys = 64;     // keys per tile: two 32-key MFMA blocks, one class per group

__device__ inline f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// two floats -> packed bf16 pair (nearest even), one v_cvt_pk_bf16_f32
__device__ inline unsigned int pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(unsigned int, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// A raw buffer resource for [p, p + bytes) held in scalar registers: the
// base and size are wave-uniform by construction, readfirstlane makes that
// explicit so loads through it need no per-lane waterfall loop.
__device__ inline __amdgpu_buffer_rsrc_t uniform_rsrc(const void* p, int bytes) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  void* q = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(q, 0, __builtin_amdgcn_readfirstlane(bytes), kBufferFlags);
}

// Combine x of lanes l and l ^ 32 (the two halves that hold one query
// column) with v_permlane32_swap, no LDS round trip.  Swapping rows 2-3 of
// (x) with rows 0-1 of (x) leaves every lane with x_lo in one result and
// x_hi in the other, so max / sum of the pair is the same in both halves.
__device__ inline float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Row (key) of register r of a 32x32 MFMA output block for lane half hh.
__device__ inline int out_row(int r, int hh) { return ((r >> 2) << 3) + (hh << 2) + (r & 3); }

// Position of key-quad kq (keys 4kq..4kq+3 of a 64-key tile) in the
// transposed V tile: inside each 16-key chunk the 4-key blocks are stored in
// the order 0, 2, 1, 3, so that lane half hh of an MFMA operand reads the
// keys {4hh..4hh+3, 8+4hh..8+4hh+3} -- the keys its S^T registers hold -- as
// one contiguous 16-byte run.
__device__ inline int vt_pos(int kq) {
  const int blk = kq & 3;
  const int nb = (blk == 1) ? 2 : (blk == 2) ? 1 : blk;
  return ((kq >> 2) << 4) + (nb << 2);
}

template <int D, int G, bool COUNT>
__global__ __launch_bounds__(kThreads, 2) void prefill_kernel(PrefillArgs a) {
  constexpr int NCH = D / 16;         // 16-dim MFMA steps
  constexpr int GC = G / 16;          // MFMA steps per group
  constexpr int NG = D / G;           // groups
  constexpr int ND = D / 32;          // 32-dim output blocks
  constexpr int KS = D + 8;           // K row stride in LDS (elements)
  constexpr int VS = kTileKeys + 8;   // V^T row stride in LDS (elements)
  constexpr int CPR = D / 8;          // 16-byte chunks per K/V row
  constexpr int KITEMS = kTileKeys * CPR / kThreads;   // K chunks per thread
  constexpr int VITEMS = 16 * CPR;                     // (key quad, chunk) items
  static_assert(KITEMS >= 1 && VITEMS <= kThreads, "tile shape");

  // two LDS stages: tile t is consumed from stage t&1 while tile t+1 is
  // written into the other one
  __shared__ __attribute__((aligned(16))) bf16 sK[2][kTileKeys * KS];
  __shared__ __attribute__((aligned(16))) bf16 sV[2][D * VS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  int bid = blockIdx.x;
  const int kvh = bid % a.Hkv;
  bid /= a.Hkv;
  const int hg = bid % a.HG;
  bid /= a.HG;
  const int b = bid % a.B;
  bid /= a.B;
  const int qblk = a.nqb - 1 - bid;
  const int n = a.n;
  const int h = kvh * a.r + hg * a.HPW + (wave % a.HPW);
  const int i0_wg = qblk * a.QB;
  // wave-uniform control values, pinned to scalar registers
  const int i0w = __builtin_amdgcn_readfirstlane(i0_wg + (wave / a.HPW) * 32);
  const bool wave_valid = i0w < n;
  const int i1w = __builtin_amdgcn_readfirstlane(min(n, i0w + 32) - 1);
  const int kend = min(n, i0_wg + a.QB);
  const int nk = __builtin_amdgcn_readfirstlane((kend + kTileKeys - 1) / kTileKeys);

  const bf16* kbase = a.k + (int64_t)b * a.ks_b + (int64_t)kvh * a.ks_h;
  const bf16* vbase = a.v + (int64_t)b * a.vs_b + (int64_t)kvh * a.vs_h;

  // Q^T operand, resident for the whole kernel: lane owns query i0w + l32,
  // dims [16c + 8hh, 16c + 8hh + 8) of MFMA step c.
  u32x4 qr[NCH];
  {
    const int i = i0w + l32;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    const bf16* qp = a.q + (int64_t)b * a.qs_b + (int64_t)i * a.qs_t + (int64_t)h * a.qs_h + hh * 8;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
      qr[c] = (i < n) ? *reinterpret_cast<const u32x4*>(qp + c * 16) : zero;
  }

  // register staging of the next K/V tile.  Tile rows are fetched with raw
  // buffer loads whose resource starts at the tile's first row and ends
  // after row n-1: rows past the end of the sequence read as zero, and the
  // per-thread byte offsets are loop invariant.
  u32x4 kreg[KITEMS];
  u32x4 vreg[4];
  const int v_kq = tid & 15;
  const int v_dc = tid >> 4;
  const bool v_active = tid < VITEMS;
  const int krow_b = (int)(a.ks_t * 2);     // bytes between consecutive keys
  const int vrow_b = (int)(a.vs_t * 2);
  int koff[KITEMS];
#pragma unroll
  for (int it = 0; it < KITEMS; ++it) {
    const int idx = tid + it * kThreads;
    koff[it] = (idx / CPR) * krow_b + (idx % CPR) * 16;
  }
  const int voff = 4 * v_kq * vrow_b + v_dc * 16;

  auto load_tile = [&](int j0) {
    const int rows = n - j0;                                  // >= 1
    const __amdgpu_buffer_rsrc_t kr =
        uniform_rsrc(kbase + (int64_t)j0 * a.ks_t, (rows - 1) * krow_b + 2 * D);
    const __amdgpu_buffer_rsrc_t vr =
        uniform_rsrc(vbase + (int64_t)j0 * a.vs_t, (rows - 1) * vrow_b + 2 * D);
#pragma unroll
    for (int it = 0; it < KITEMS; ++it)
      kreg[it] = __builtin_amdgcn_raw_buffer_load_b128(kr, koff[it], 0, 0);
    if (v_active) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        vreg[q4] = __builtin_amdgcn_raw_buffer_load_b128(vr, voff + q4 * vrow_b, 0, 0);
    }
  };

  auto store_tile = [&](int stage) {
    bf16* k_s = sK[stage];
    bf16* v_s = sV[stage];
#pragma unroll
    for (int it = 0; it < KITEMS; ++it) {
      const int idx = tid + it * kThreads;
      const int key = idx / CPR;
      const int dc = idx % CPR;
      *reinterpret_cast<u32x4*>(&k_s[key * KS + dc * 8]) = kreg[it];
    }
    if (v_active) {
      // vreg[q] holds dims [8dc, 8dc+8) of key 4kq+q as 4 dwords of 2 dims;
      // write, for every dim, the 4 keys as one 8-byte run of V^T.
      const int pos = vt_pos(v_kq);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const unsigned int w0 = vreg[0][e], w1 = vreg[1][e], w2 = vreg[2][e], w3 = vreg[3][e];
        u32x2 even, odd;
        even[0] = __builtin_amdgcn_perm(w1, w0, 0x05040100u);   // (w0.lo, w1.lo)
        even[1] = __builtin_amdgcn_perm(w3, w2, 0x05040100u);
        odd[0] = __builtin_amdgcn_perm(w1, w0, 0x07060302u);    // (w0.hi, w1.hi)
        odd[1] = __builtin_amdgcn_perm(w3, w2, 0x07060302u);
        const int d = v_dc * 8 + 2 * e;
        *reinterpret_cast<u32x2*>(&v_s[d * VS + pos]) = even;
        *reinterpret_cast<u32x2*>(&v_s[(d + 1) * VS + pos]) = odd;
      }
    }
  };

  float m_i = -INFINITY;   // running max (log2 domain), possibly stale by < 8
  float l_i = 0.f;         // running sum (this lane's half of the keys)
  f32x16 o[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;

  unsigned int cnt[NG][3];
  unsigned int cnt_vis = 0;
  if (COUNT) {
#pragma unroll
    for (int g = 0; g < NG; ++g) cnt[g][0] = cnt[g][1] = cnt[g][2] = 0;
  }

  const float sl2 = a.scale_log2;
  const f32x16 zero16 = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};

  load_tile(0);
  store_tile(0);
  if (nk > 1) load_tile(kTileKeys);
  __syncthreads();

  for (int it = 0; it < nk; ++it) {
    const int j0 = it * kTileKeys;
    const int stage = it & 1;
    if (wave_valid && j0 <= i1w) {
      // ---- classify the (32 queries x 64 keys) tile ----
      const int j1 = min(n - 1, j0 + kTileKeys - 1);
      const int lD = max(0, i0w - j1);
      const int rD = i1w - j0;
      // cutoffs are non-decreasing: splitL / splitR = 1 + last group below
      int sL = 0, sR = 0;
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        sL = (a.cut[g] < lD) ? g + 1 : sL;
        sR = (a.cut[g] < rD) ? g + 1 : sR;
      }
      sL = __builtin_amdgcn_readfirstlane(sL);
      sR = __builtin_amdgcn_readfirstlane(sR);
      if (COUNT) {
        ++cnt_vis;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          cnt[g][0] += (g < sL);
          cnt[g][1] += (g >= sL && g < sR);
          cnt[g][2] += (g >= sR);
        }
      }

      // ---- S^T = K Q^T: full groups [sR, NG) as one chain, highest first ----
      const bf16* k0 = &sK[stage][l32 * KS + hh * 8];
      const bf16* k1 = k0 + 32 * KS;
      f32x16 s0, s1;
      if (sR < NG) {
        {
          constexpr int c0 = (NG - 1) * GC;
          s0 = mfma32(*reinterpret_cast<const u32x4*>(k0 + c0 * 16), qr[c0], zero16);
          s1 = mfma32(*reinterpret_cast<const u32x4*>(k1 + c0 * 16), qr[c0], zero16);
#pragma unroll
          for (int c = 1; c < GC; ++c) {
            s0 = mfma32(*reinterpret_cast<const u32x4*>(k0 + (c0 + c) * 16), qr[c0 + c], s0);
            s1 = mfma32(*reinterpret_cast<const u32x4*>(k1 + (c0 + c) * 16), qr[c0 + c], s1);
          }
        }
#pragma unroll
        for (int g = NG - 2; g >= 0; --g) {
          if (g < sR) break;
#pragma unroll
          for (int c = 0; c < GC; ++c) {
            const int cc = g * GC + c;
            s0 = mfma32(*reinterpret_cast<const u32x4*>(k0 + cc * 16), qr[cc], s0);
            s1 = mfma32(*reinterpret_cast<const u32x4*>(k1 + cc * 16), qr[cc], s1);
          }
        }
      } else {
        s0 = zero16;
        s1 = zero16;
      }

      // ---- partial groups [sL, sR): compute, mask dist <= cutoff, add ----
      if (sL < sR) {
        const int base = (i0w + l32) - j0;     // dist = base - (32kb + out_row(r))
#pragma unroll
        for (int g = NG - 1; g >= 0; --g) {
          if (g >= sR || g < sL) continue;
          const int cg = a.cut[g];
          f32x16 t = zero16;
#pragma unroll
          for (int c = 0; c < GC; ++c) {
            const int cc = g * GC + c;
            t = mfma32(*reinterpret_cast<const u32x4*>(k0 + cc * 16), qr[cc], t);
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) s0[r] += (base - out_row(r, hh) <= cg) ? t[r] : 0.f;
          t = zero16;
#pragma unroll
          for (int c = 0; c < GC; ++c) {
            const int cc = g * GC + c;
            t = mfma32(*reinterpret_cast<const u32x4*>(k1 + cc * 16), qr[cc], t);
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) s1[r] += (base - 32 - out_row(r, hh) <= cg) ? t[r] : 0.f;
        }
      }

      // ---- causal mask on tiles that reach past the wave's first query ----
      if (j0 + kTileKeys - 1 > i0w) {
        const int base = (i0w + l32) - j0;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if (out_row(r, hh) > base) s0[r] = -INFINITY;
          if (32 + out_row(r, hh) > base) s1[r] = -INFINITY;
        }
      }

      // ---- online softmax, log2 domain; rescale O only when the running
      //      max grows by more than 8 (so every p stays <= 2^8) ----
      float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(fmaxf(mx, s0[r]), s1[r]);   // v_max3 chain
      mx = halves_max(mx);
      const float m_cand = mx * sl2;
      if (__any(m_cand > m_i + 8.f)) {
        const float m_new = fmaxf(m_i, m_cand);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_i - m_use);
        l_i *= alpha;
#pragma unroll
        for (int db = 0; db < ND; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
        m_i = m_use;
      }
      u32x4 p[4];
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int r = 8 * c + 2 * w;
          const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[r], sl2, -m_i));
          const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[r + 1], sl2, -m_i));
          const float f0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[r], sl2, -m_i));
          const float f1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[r + 1], sl2, -m_i));
          l_i += (e0 + e1) + (f0 + f1);
          p[c][w] = pack_bf16x2(e0, e1);
          p[2 + c][w] = pack_bf16x2(f0, f1);
        }

      // ---- O^T += V^T P^T ----
      const bf16* vs = &sV[stage][l32 * VS + hh * 8];
#pragma unroll
      for (int kc = 0; kc < 4; ++kc)
#pragma unroll
        for (int db = 0; db < ND; ++db) {
          const u32x4 va = *reinterpret_cast<const u32x4*>(vs + db * 32 * VS + kc * 16);
          o[db] = mfma32(va, p[kc], o[db]);
        }
    }

    // ---- stage the next tile; prefetch the one after ----
    if (it + 1 < nk) store_tile(stage ^ 1);
    if (it + 2 < nk) load_tile((it + 2) * kTileKeys);
    __syncthreads();
  }

  if (wave_valid) {
    const float l_tot = halves_sum(l_i);
    const int i = i0w + l32;
    if (i < n) {
      const float inv = 1.f / l_tot;
      bf16* op = a.o + (int64_t)b * a.os_b + (int64_t)i * a.os_t + (int64_t)h * a.os_h + hh * 4;
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          u32x2 w;
          w[0] = pack_bf16x2(o[db][4 * r4] * inv, o[db][4 * r4 + 1] * inv);
          w[1] = pack_bf16x2(o[db][4 * r4 + 2] * inv, o[db][4 * r4 + 3] * inv);
          *reinterpret_cast<u32x2*>(op + db * 32 + r4 * 8) = w;
        }
      if (a.lse && hh == 0)
        a.lse[((int64_t)b * a.Hq + h) * n + i] = (m_i + __log2f(l_tot)) * 0.69314718055994531f;
    }
    if (COUNT && lane == 0) {
#pragma unroll
      for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int c = 0; c < 3; ++c)
          if (cnt[g][c]) atomicAdd(&a.counters[3 * g + c], (unsigned long long)cnt[g][c]);
      if (cnt_vis) atomicAdd(&a.counters[3 * NG], (unsigned long long)cnt_vis);
    }
  }
}

template <int D, int G>
hipError_t launch_dg(const PrefillArgs& a, bool count, hipStream_t s) {
  const long long blocks = (long long)a.B * a.Hkv * a.HG * a.nqb;
  if (blocks <= 0) return hipSuccess;
  if (count)
    hipLaunchKernelGGL((prefill_kernel<D, G, true>), dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((prefill_kernel<D, G, false>), dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, int d_h, int G, bool count, hipStream_t s) {
  if (d_h == 128 && G == 16) return launch_dg<128, 16>(a, count, s);
  if (d_h == 128 && G == 32) return launch_dg<128, 32>(a, count, s);
  if (d_h == 64 && G == 16) return launch_dg<64, 16>(a, count, s);
  if (d_h == 64 && G == 32) return launch_dg<64, 32>(a, count, s);
  return hipErrorInvalidValue;
}

}  // namespace wp
