// WavePrune causal prefill attention for gfx950 (grouped rule).
//
// Method: every RoPE channel adds to the QK logit only while the distance is
// within its cutoff; pruned terms are 0 and the key stays in the softmax
// (WavePrune reading notes on cc.laoqi.cc, section 2.1, Eq. (6)).  Head dims
// are grouped (G = 16 or 32) and a group uses the largest cutoff inside it
// (section 2.3, Eq. (8)).  Each (32-query x 32-key) tile is classified per
// group from its distance range [l_D, r_D]: skip, partial or full
// (section 2.3 table).  Because the cutoffs are non-decreasing two split
// points describe a tile: groups [0, splitL) skip, [splitL, splitR) partial,
// [splitR, ng) full (section 2.3, the paragraph on splitL/splitR).
//
// gfx950 design (not the pages' A100 design):
//  * The logits are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: one MFMA contracts exactly 16 head dims, so a
//    G = 16 group is one MFMA per 32x32 tile and G = 32 is two.  In S^T the
//    lane owns one query column, so row max / row sum need one cross-half
//    exchange only, and the probabilities are already laid out as the B
//    operand of O^T = V^T P^T.
//  * Skipped groups issue no MFMA; full groups chain into one accumulator
//    (the "suffix" GEMM); a partial group gets its own accumulator, is masked
//    with dist <= cutoff, then added.  The branches are wave-uniform scalar
//    branches, so no per-(splitL, splitR) code specialization is needed.
//  * A workgroup is 4 waves that share one kv head and one key range: with
//    GQA ratio >= 4 the waves are 4 query heads over the same 32 queries
//    (identical tile classes, K/V staged once in LDS for all four).
//  * K is staged row-major in LDS (row pad 16 B: conflict-free 16-byte MFMA
//    operand reads); V is written transposed (V^T) with a key permutation
//    that matches the S^T register layout, so both MFMA operands of P.V are
//    single 16-byte LDS reads.  The next K/V tile is prefetched into
//    registers while the current one is consumed.
//  * Workgroups run heaviest (last query blocks) first; kv head is the
//    fastest-varying block index so that on 8 kv heads each XCD (blocks are
//    dealt round-robin to the 8 XCDs) keeps one kv head's K/V in its L2.
#include "wp_internal.h"

namespace wp {

namespace {

constexpr int kThreads = 256;
constexpr int kTileKeys = 64;     // keys per LDS tile (two 32-key MFMA blocks)

__device__ inline f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ inline unsigned int pack_bf16x2(float lo, float hi) {
  const __bf16 a = static_cast<__bf16>(lo);
  const __bf16 b = static_cast<__bf16>(hi);
  return (unsigned int)__builtin_bit_cast(unsigned short, a) |
         ((unsigned int)__builtin_bit_cast(unsigned short, b) << 16);
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

  __shared__ __attribute__((aligned(16))) bf16 sK[kTileKeys * KS];
  __shared__ __attribute__((aligned(16))) bf16 sV[D * VS];

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
  const int i0w = i0_wg + (wave / a.HPW) * 32;
  const bool wave_valid = i0w < n;
  const int i1w = min(n, i0w + 32) - 1;
  const int kend = min(n, i0_wg + a.QB);
  const int nk = (kend + kTileKeys - 1) / kTileKeys;

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

  // register staging of the next K/V tile
  u32x4 kreg[KITEMS];
  u32x4 vreg[4];
  const int v_kq = tid & 15;
  const int v_dc = tid >> 4;
  const bool v_active = tid < VITEMS;

  auto load_tile = [&](int j0) {
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int it = 0; it < KITEMS; ++it) {
      const int idx = tid + it * kThreads;
      const int key = idx / CPR;
      const int dc = idx % CPR;
      const int j = j0 + key;
      kreg[it] = (j < n) ? *reinterpret_cast<const u32x4*>(kbase + (int64_t)j * a.ks_t + dc * 8)
                         : zero;
    }
    if (v_active) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int j = j0 + 4 * v_kq + q4;
        vreg[q4] = (j < n) ? *reinterpret_cast<const u32x4*>(vbase + (int64_t)j * a.vs_t + v_dc * 8)
                           : zero;
      }
    }
  };

  auto store_tile = [&]() {
#pragma unroll
    for (int it = 0; it < KITEMS; ++it) {
      const int idx = tid + it * kThreads;
      const int key = idx / CPR;
      const int dc = idx % CPR;
      *reinterpret_cast<u32x4*>(&sK[key * KS + dc * 8]) = kreg[it];
    }
    if (v_active) {
      // vreg[q] holds dims [8dc, 8dc+8) of key 4kq+q as 4 dwords of 2 dims;
      // write, for every dim, the 4 keys as one 8-byte run of V^T.
      const int pos = vt_pos(v_kq);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const unsigned int w0 = vreg[0][e], w1 = vreg[1][e], w2 = vreg[2][e], w3 = vreg[3][e];
        u32x2 even, odd;
        even[0] = (w0 & 0xffffu) | (w1 << 16);
        even[1] = (w2 & 0xffffu) | (w3 << 16);
        odd[0] = (w0 >> 16) | (w1 & 0xffff0000u);
        odd[1] = (w2 >> 16) | (w3 & 0xffff0000u);
        const int d = v_dc * 8 + 2 * e;
        *reinterpret_cast<u32x2*>(&sV[d * VS + pos]) = even;
        *reinterpret_cast<u32x2*>(&sV[(d + 1) * VS + pos]) = odd;
      }
    }
  };

  float m_i = -INFINITY;   // running max, log2 domain
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
  load_tile(0);

  for (int it = 0; it < nk; ++it) {
    const int j0 = it * kTileKeys;
    __syncthreads();
    store_tile();
    __syncthreads();
    if (it + 1 < nk) load_tile(j0 + kTileKeys);
    if (!wave_valid || j0 > i1w) continue;

    f32x16 s[2];
    bool vis[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int jb0 = j0 + 32 * kb;
      vis[kb] = jb0 <= i1w;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
      if (!vis[kb]) continue;
      const int jb1 = min(n - 1, jb0 + 31);
      const int lD = max(0, i0w - jb1);
      const int rD = i1w - jb0;
      int sL = 0, sR = 0;
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        sL += a.cut[g] < lD;
        sR += a.cut[g] < rD;
      }
      if (COUNT) {
        ++cnt_vis;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          cnt[g][0] += (g < sL);
          cnt[g][1] += (g >= sL && g < sR);
          cnt[g][2] += (g >= sR);
        }
      }
      const bf16* krow = &sK[(32 * kb + l32) * KS + hh * 8];
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        if (g < sL) continue;                       // skip: no MFMA
        if (g >= sR) {                              // full: chain into S
#pragma unroll
          for (int c = 0; c < GC; ++c) {
            const u32x4 ka = *reinterpret_cast<const u32x4*>(krow + (g * GC + c) * 16);
            s[kb] = mfma32(ka, qr[g * GC + c], s[kb]);
          }
        } else {                                    // partial: compute, mask, add
          f32x16 t;
#pragma unroll
          for (int r = 0; r < 16; ++r) t[r] = 0.f;
#pragma unroll
          for (int c = 0; c < GC; ++c) {
            const u32x4 ka = *reinterpret_cast<const u32x4*>(krow + (g * GC + c) * 16);
            t = mfma32(ka, qr[g * GC + c], t);
          }
          const int base = (i0w + l32) - jb0;       // dist = base - out_row(r)
          const int cg = a.cut[g];
#pragma unroll
          for (int r = 0; r < 16; ++r)
            s[kb][r] += (base - out_row(r, hh) <= cg) ? t[r] : 0.f;
        }
      }
      if (jb0 + 31 > i0w) {                         // crosses the diagonal
        const int base = (i0w + l32) - jb0;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (out_row(r, hh) > base) s[kb][r] = -INFINITY;
      }
    }

    // online softmax (log2 domain, scale folded into the exponent)
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
      if (vis[kb]) {
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_i, mx * sl2);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_i - m_use);
    l_i *= alpha;
    u32x4 p[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (!vis[kb]) continue;
      float e[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        e[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], sl2, -m_use));
        l_i += e[r];
      }
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int w = 0; w < 4; ++w)
          p[2 * kb + c][w] = pack_bf16x2(e[8 * c + 2 * w], e[8 * c + 2 * w + 1]);
    }
    if (__any(m_new > m_i)) {
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
    }
    m_i = m_new;

    // O^T += V^T P^T
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      if (!vis[kc >> 1]) continue;
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        const u32x4 va = *reinterpret_cast<const u32x4*>(&sV[(db * 32 + l32) * VS + kc * 16 + hh * 8]);
        o[db] = mfma32(va, p[kc], o[db]);
      }
    }
  }

  if (wave_valid) {
    const float l_tot = l_i + __shfl_xor(l_i, 32);
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
