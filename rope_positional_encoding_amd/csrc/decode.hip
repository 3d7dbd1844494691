// WavePrune decode attention for gfx950: one new query token per sequence
// against a KV cache, split over the keys, then merged.
//
// Rule: a head-dim group adds to the logit only while the query-key distance
// is within its cutoff; the key stays in the softmax (WavePrune reading notes
// on cc.laoqi.cc, section 2.1, Eq. (6); grouped cutoffs, section 2.3,
// Eq. (8)).  In decode a skipped group's K columns are never read
// (section 2.3 table: skip = less QK and no K-cache read for the group; the
// system section 4.6 attributes the decode gain to these K reads).
//
// gfx950 design:
//  * HBM-bound: the aim is to stream the kept K bytes and all V bytes once.
//    A workgroup (4 waves) owns one (sequence, kv head, split); split s of S
//    takes the 32-key blocks s, s + S, s + 2S, ... so that all splits of a
//    sequence advance through the cache together.  Each wave walks its own
//    blocks independently (no barriers in the loop) and keeps its own
//    online-softmax state for the GQA heads.
//  * QK on v_mfma_f32_16x16x32_bf16 with the keys as rows: each lane loads
//    16 contiguous bytes of one key row straight from HBM into the MFMA A
//    operand; the GQA heads are the B columns, held in registers: up to 16,
//    or up to 32 as two head sets that share every K and V operand.  Lanes
//    whose 8 dims belong to a skipped group issue no load.
//  * P.V on the same MFMA as O^T = V^T P^T: the probabilities are already in
//    the B layout; V is staged through a per-wave LDS tile written transposed
//    (keys permuted to match), so the A operand is one 16-byte LDS read.
//  * The 4 waves merge through LDS at the end; a second kernel merges the
//    splits (log-sum-exp weighted), one wave per (sequence, query head).
#include <mutex>

#include "wp_device.h"
#include "wp_internal.h"

namespace wp {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;

__device__ inline f32x4 mfma16(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Position of key-quad kq (keys 4kq..4kq+3 of a 32-key block) inside the
// transposed V tile.  Lane quarter q of the P.V MFMA owns keys
// {4q..4q+3} (block rows of the first 16 keys) and {16+4q..16+4q+3}; they
// are stored at positions [8q, 8q+8).
__device__ inline int vt_pos32(int kq) { return kq < 4 ? 8 * kq : 8 * (kq - 4) + 4; }

// j mod c for 0 <= j < 2^24 and 1 <= c < 2^24, with rc = 1/c rounded to
// float: the float quotient is off by at most one, which the two
// corrections remove.
__device__ inline int mod_small(int j, int c, float rc) {
  int r = j - (int)((float)j * rc) * c;
  r += (r < 0) ? c : 0;
  r -= (r >= c) ? c : 0;
  return r;
}

// HS head sets of 16: a launch takes up to 16 * HS query heads per kv head,
// the MFMA columns of set hs being heads 16 hs .. 16 hs + 15; the K and V
// operands of a block serve every set.
template <int D, int G, bool COUNT, bool COMPACT, int HS>
__global__ __launch_bounds__(kThreads, 2) void decode_split_kernel(DecodeArgs a) {
  constexpr int NP = D / 32;          // 32-dim MFMA steps of QK
  constexpr int NG = D / G;           // groups
  constexpr bool FINE = G < 16;       // a lane's 8 dims may span several groups (G = 2: channels)
  static_assert(!(FINE && COMPACT), "the compact K store takes groups of 16 or 32 dims");
  constexpr int ND = D / 16;          // 16-dim output blocks
  constexpr int VS = 32 + 8;          // V^T row stride in LDS (elements)
  constexpr int VITEMS = 8 * (D / 8) / 64;   // (key quad, chunk) items per lane
  static_assert(VITEMS >= 1, "tile shape");

  __shared__ __attribute__((aligned(16))) bf16 sV[kWaves][D * VS];
  __shared__ float sM[kWaves][16];
  __shared__ float sL[kWaves][16];
  static_assert(HS == 1 || HS == 2, "head sets");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n16 = lane & 15;     // MFMA column: GQA head (B/C) or row (A)
  const int q4 = lane >> 4;      // lane quarter

  int bid = blockIdx.x;
  const int kvh = bid % a.Hkv;
  bid /= a.Hkv;
  const int split = bid % a.S;
  const int b = bid / a.S;

  const int L = __builtin_amdgcn_readfirstlane(min(a.cache_len[b], a.Lmax));
  const int qp = __builtin_amdgcn_readfirstlane(a.q_pos[b]);

  // Q^T operand of head set hs: column n16 = head kvh*rs + 16hs + n16 (zero
  // from r on), dims [32p + 8q4, 32p + 8q4 + 8) of step p.
  u32x4 qr[HS][NP];
#pragma unroll
  for (int hs = 0; hs < HS; ++hs) {
    const u32x4 zero = {0u, 0u, 0u, 0u};
    const int hd = 16 * hs + n16;
    const bf16* qb = a.q + (int64_t)b * a.qs_b + (int64_t)(kvh * a.rs + hd) * a.qs_h + q4 * 8;
#pragma unroll
    for (int p = 0; p < NP; ++p)
      qr[hs][p] = (hd < a.r) ? *reinterpret_cast<const u32x4*>(qb + p * 32) : zero;
  }

  // K / V of this (sequence, kv head) through raw buffer resources.  For the
  // full cache each 32-key block gets its own resources, from its first key
  // to min(L, block end) - 1, so offsets stay within one block (32-bit,
  // whatever the cache length): rows past the cache length read as zero, and
  // a lane whose 8 dims belong to a skipped group gets an out-of-range
  // offset, so it fetches nothing and reads zero -- no branches around the
  // loads.  The compact store is one resource per (sequence, kv head).
  const int krow_b = (int)(a.ks_t * 2);
  const int vrow_b = (int)(a.vs_t * 2);
  const bf16* kseq = a.k + (int64_t)b * a.ks_b + (int64_t)kvh * a.ks_h;
  const bf16* vseq = a.v + (int64_t)b * a.vs_b + (int64_t)kvh * a.vs_h;
  const __amdgpu_buffer_rsrc_t kstore = uniform_rsrc(kseq, COMPACT ? 2 * a.kstore_elems : 0);
  // compact store: ring size, its reciprocal and the ring's byte offset for
  // the group this lane reads in QK step p.  The kernel arguments are read
  // with uniform indices only (a lane-dependent index would turn them into
  // per-lane memory loads, whose waits would also drain the K/V loads in
  // flight).
  int kcap_p[NP], kbase_p[NP];
  float rcap_p[NP];
  if (COMPACT) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int gl = (32 * p) / G, gh = (32 * p + 24) / G;
      const bool lo = ((32 * p + 8 * q4) / G) == gl;
      kcap_p[p] = lo ? a.kcap[gl] : a.kcap[gh];
      kbase_p[p] = (lo ? a.koff[gl] : a.koff[gh]) * 2;
      rcap_p[p] = 1.0f / (float)kcap_p[p];
    }
  }
  constexpr int kOut = 0x7ffffff0;    // any offset >= the resource size

  bf16* sv = sV[wave];
  float m_i[HS], l_i[HS];
  f32x4 o[HS][ND];
#pragma unroll
  for (int hs = 0; hs < HS; ++hs) {
    m_i[hs] = -INFINITY;
    l_i[hs] = 0.f;
#pragma unroll
    for (int db = 0; db < ND; ++db) o[hs][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Tile-class counters: per group in registers for coarse groups; for fine
  // groups (up to 64) a workgroup histogram of splitL / splitR in LDS,
  // turned into per-group counts at the end.
  constexpr int CNG = FINE ? 1 : NG;
  unsigned int cnt[CNG][3];
  unsigned int cnt_vis = 0;
  __shared__ unsigned int s_hist[(COUNT && FINE) ? 2 * (NG + 1) : 1];
  // Fine groups: the cutoff table in LDS, and split points carried from
  // block to block (a wave meets its key blocks in ascending order, so the
  // distances and the split points only decrease).  cL / cR hold the cutoff
  // of group fL - 1 / fR - 1 in scalar registers, so a block whose split
  // points do not move reads no LDS.
  __shared__ int s_cut[FINE ? NG : 1];
  int fL = NG, fR = NG;
  int cL = 0, cR = 0;
  if (COUNT) {
#pragma unroll
    for (int g = 0; g < CNG; ++g) cnt[g][0] = cnt[g][1] = cnt[g][2] = 0;
    if constexpr (FINE) {
      if (tid < 2 * (NG + 1)) s_hist[tid] = 0;
    }
  }
  if constexpr (FINE) {
    if (tid < NG) s_cut[tid] = a.cut[tid];
    __syncthreads();
    cL = cR = __builtin_amdgcn_readfirstlane(s_cut[NG - 1]);
  }
  const float sl2 = a.scale_log2;

  struct Regs {
    u32x4 k[2][NP];
    u32x4 v[VITEMS][4];
  };

  // classes of the key block starting at jb: skip groups [0, sL), partial
  // [sL, sR), full [sR, NG)
  auto classify = [&](int jb, int& sL, int& sR) {
    const int jb1 = min(L, jb + 32) - 1;
    const int lD = __builtin_amdgcn_readfirstlane(qp - jb1);   // wave-uniform
    const int rD = __builtin_amdgcn_readfirstlane(qp - jb);
    if constexpr (FINE) {
      // idempotent for one block, so the load and the compute of a block
      // may both call it
      auto cut_at = [&](int g) { return __builtin_amdgcn_readfirstlane(s_cut[g]); };
      while (fL > 0 && cL >= lD) {
        --fL;
        cL = fL > 0 ? cut_at(fL - 1) : 0;
      }
      while (fR > 0 && cR >= rD) {
        --fR;
        cR = fR > 0 ? cut_at(fR - 1) : 0;
      }
      sL = __builtin_amdgcn_readfirstlane(fL);
      sR = __builtin_amdgcn_readfirstlane(fR);
    } else {
      sL = 0;
      sR = 0;
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        sL = (a.cut[g] < lD) ? g + 1 : sL;
        sR = (a.cut[g] < rD) ? g + 1 : sR;
      }
      sL = __builtin_amdgcn_readfirstlane(sL);
      sR = __builtin_amdgcn_readfirstlane(sR);
    }
  };

  // issue every HBM load of one block: the kept K columns and all of V
  auto load_block = [&](Regs& R, int jb) {
    int sL, sR;
    classify(jb, sL, sR);
    const int rows = min(32, L - jb);          // >= 1
    const __amdgpu_buffer_rsrc_t krs =
        COMPACT ? kstore : uniform_rsrc(kseq + (int64_t)jb * a.ks_t, (rows - 1) * krow_b + 2 * D);
    const __amdgpu_buffer_rsrc_t vrs = uniform_rsrc(vseq + (int64_t)jb * a.vs_t, (rows - 1) * vrow_b + 2 * D);
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const int j = jb + 16 * blk + n16;
      const int row = (16 * blk + n16) * krow_b;     // within the block
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const int dim = 32 * p + 8 * q4;
        const int g = (dim + 7) / G;              // the last group of this lane's 8 dims
        int off;
        if (COMPACT) {
          const int slot = mod_small(j, kcap_p[p], rcap_p[p]);
          off = (g >= sL && j < L) ? kbase_p[p] + (slot * G + dim % G) * 2 : kOut;
        } else {
          off = (g >= sL) ? row + dim * 2 : kOut;
        }
        R.k[blk][p] = __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, 0);
      }
    }
#pragma unroll
    for (int it = 0; it < VITEMS; ++it) {
      const int kq = lane & 7;
      const int dc = (lane >> 3) + 8 * it;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        R.v[it][e] = __builtin_amdgcn_raw_buffer_load_b128(vrs, (4 * kq + e) * vrow_b + dc * 16, 0, 0);
    }
  };

  auto compute_block = [&](Regs& R, int jb) {
    int sL, sR;
    classify(jb, sL, sR);
    const int jb1 = min(L, jb + 32) - 1;
    if (COUNT) {
      ++cnt_vis;
      if constexpr (FINE) {
        if (lane == 0) {
          atomicAdd(&s_hist[sL], 1u);
          atomicAdd(&s_hist[NG + 1 + sR], 1u);
        }
      } else {
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          cnt[g][0] += (g < sL);
          cnt[g][1] += (g >= sL && g < sR);
          cnt[g][2] += (g >= sR);
        }
      }
    }
    const u32x4 zero = {0u, 0u, 0u, 0u};

    // ---- S^T = K Q^T per 16-key block and head set, group by group ----
    f32x4 s[HS][2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
      for (int hs = 0; hs < HS; ++hs) s[hs][blk] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const int g_lo = (32 * p) / G;             // groups covered by step p
        const int g_hi = (32 * p + 31) / G;
        if (g_hi < sL) continue;                   // every lane skipped
        const int g = (32 * p + 8 * q4) / G;
        // group of operand word w (dims 32p + 8q4 + 2w, +1)
        auto grp = [&](int w) { return (32 * p + 8 * q4 + 2 * w) / G; };
        if (g_lo >= sR) {                          // all full: skipped lanes read zero
#pragma unroll
          for (int hs = 0; hs < HS; ++hs) s[hs][blk] = mfma16(R.k[blk][p], qr[hs][p], s[hs][blk]);
          continue;
        }
        const bool any_full = g_hi >= sR;          // the step's last group is full
        if (any_full) {
          const u32x4 op = FINE ? keep_words(R.k[blk][p], [&](int w) { return grp(w) >= sR; })
                                : ((g >= sR) ? R.k[blk][p] : zero);
#pragma unroll
          for (int hs = 0; hs < HS; ++hs) s[hs][blk] = mfma16(op, qr[hs][p], s[hs][blk]);
        }
        if constexpr (FINE) {
          // a runtime loop over just this step's partial groups: unrolled
          // over all 32/G groups of every step the kernel outgrows the
          // instruction cache
#pragma unroll 1
          for (int gg = max(g_lo, sL); gg < min(g_hi + 1, sR); ++gg) {
            const u32x4 op = keep_words(R.k[blk][p], [&](int w) { return grp(w) == gg; });
            const int cg = __builtin_amdgcn_readfirstlane(s_cut[gg]);
#pragma unroll
            for (int hs = 0; hs < HS; ++hs) {
              const f32x4 t = mfma16(op, qr[hs][p], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int j = jb + 16 * blk + 4 * q4 + r;
                s[hs][blk][r] += (qp - j <= cg) ? t[r] : 0.f;
              }
            }
          }
        } else {
#pragma unroll
          for (int gg = g_lo; gg <= g_hi; ++gg) {
            if (gg < sL || gg >= sR) continue;     // only partial groups
            const u32x4 op = (g == gg) ? R.k[blk][p] : zero;
            const int cg = a.cut[gg];
#pragma unroll
            for (int hs = 0; hs < HS; ++hs) {
              const f32x4 t = mfma16(op, qr[hs][p], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int j = jb + 16 * blk + 4 * q4 + r;
                s[hs][blk][r] += (qp - j <= cg) ? t[r] : 0.f;
              }
            }
          }
        }
      }
      if (jb + 32 > L) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = jb + 16 * blk + 4 * q4 + r;
#pragma unroll
          for (int hs = 0; hs < HS; ++hs)
            if (j > jb1) s[hs][blk][r] = -INFINITY;
        }
      }
    }

    // ---- V^T into this wave's LDS tile ----
#pragma unroll
    for (int it = 0; it < VITEMS; ++it) {
      const int kq = lane & 7;
      const int dc = (lane >> 3) + 8 * it;
      const int pos = vt_pos32(kq);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const unsigned int w0 = R.v[it][0][e], w1 = R.v[it][1][e], w2 = R.v[it][2][e], w3 = R.v[it][3][e];
        u32x2 even, odd;
        even[0] = __builtin_amdgcn_perm(w1, w0, 0x05040100u);   // (w0.lo, w1.lo)
        even[1] = __builtin_amdgcn_perm(w3, w2, 0x05040100u);
        odd[0] = __builtin_amdgcn_perm(w1, w0, 0x07060302u);    // (w0.hi, w1.hi)
        odd[1] = __builtin_amdgcn_perm(w3, w2, 0x07060302u);
        const int d = dc * 8 + 2 * e;
        *reinterpret_cast<u32x2*>(&sv[d * VS + pos]) = even;
        *reinterpret_cast<u32x2*>(&sv[(d + 1) * VS + pos]) = odd;
      }
    }

    // ---- online softmax over this block (log2 domain).  The running max m_i
    //      (per head) is refreshed, and O and l rescaled, only when some
    //      head's max grows by more than 8, so every probability stays below
    //      2^8; O / l and the partial (m, l) pairs are unaffected. ----
    u32x4 pb[HS];
#pragma unroll
    for (int hs = 0; hs < HS; ++hs) {
      const f32x4* sh = s[hs];
      float mx = fmaxf(fmaxf(fmaxf(sh[0][0], sh[0][1]), fmaxf(sh[0][2], sh[0][3])),
                       fmaxf(fmaxf(sh[1][0], sh[1][1]), fmaxf(sh[1][2], sh[1][3])));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_cand = mx * sl2;
      if (__any(m_cand > m_i[hs] + 8.f)) {
        const float m_new = fmaxf(m_i[hs], m_cand);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_i[hs] - m_use);
        l_i[hs] *= alpha;
#pragma unroll
        for (int db = 0; db < ND; ++db) o[hs][db] *= alpha;
        m_i[hs] = m_use;
      }
      float e[8];
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          e[4 * blk + r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sh[blk][r], sl2, -m_i[hs]));
          l_i[hs] += e[4 * blk + r];
        }
#pragma unroll
      for (int w = 0; w < 4; ++w) pb[hs][w] = pack_bf16x2(e[2 * w], e[2 * w + 1]);
    }

    // the V^T tile was written by other lanes of this wave
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int db = 0; db < ND; ++db) {
      const u32x4 va = *reinterpret_cast<const u32x4*>(&sv[(16 * db + n16) * VS + 8 * q4]);
#pragma unroll
      for (int hs = 0; hs < HS; ++hs) o[hs][db] = mfma16(va, pb[hs], o[hs][db]);
    }
    // the next block overwrites the tile only after these reads completed
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  };

  // ---- this split's key blocks are split, split + S, split + 2S, ... and
  //      wave w takes every 4th of them, so the S workgroups of a (sequence,
  //      kv head) sweep the cache together, block by block: at any moment
  //      the running workgroups read a few dense address ranges (friendly to
  //      the DRAM pages), and near and far keys are spread evenly over the
  //      splits.  One register set per wave, so that the kernel fits two
  //      waves per SIMD (a second set, with the next block's loads in
  //      flight during compute, needed AGPRs and ran 4% slower). ----
  const int kStride = 32 * a.S * kWaves;
  Regs RA;
  for (int jb = 32 * (split + a.S * wave); jb < L; jb += kStride) {
    load_block(RA, jb);
    compute_block(RA, jb);
  }

  // ---- merge the 4 waves of this split through LDS, one head set at a
  //      time (the set's O tiles reuse the V^T tiles' LDS) ----
  float* sO = reinterpret_cast<float*>(&sV[0][0]);   // [kWaves][16][D]
  static_assert(sizeof(float) * kWaves * 16 * D <= sizeof(bf16) * kWaves * D * VS, "LDS reuse");
#pragma unroll
  for (int hs = 0; hs < HS; ++hs) {
    const float l_tot = l_i[hs] + __shfl_xor(l_i[hs], 16);
    const float l_all = l_tot + __shfl_xor(l_tot, 32);
    // every wave is done with its V^T tile (first set) or with the previous
    // set's merge reads before the LDS is written again
    __syncthreads();
    if (q4 == 0) {
      sM[wave][n16] = m_i[hs];
      sL[wave][n16] = l_all;
    }
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) sO[(wave * 16 + n16) * D + 16 * db + 4 * q4 + r] = o[hs][db][r];
    __syncthreads();

    const int r_set = min(16, a.r - 16 * hs);     // heads of this set in the launch
    for (int idx = tid; idx < r_set * D; idx += kThreads) {
      const int hd = idx / D;
      const int d = idx - hd * D;
      float mm = -INFINITY;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) mm = fmaxf(mm, sM[w][hd]);
      float acc = 0.f, lsum = 0.f;
      if (mm != -INFINITY) {
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          const float sc = __builtin_amdgcn_exp2f(sM[w][hd] - mm);
          acc += sc * sO[(w * 16 + hd) * D + d];
          lsum += sc * sL[w][hd];
        }
      }
      const int h = kvh * a.r + 16 * hs + hd;
      const int64_t pi = ((int64_t)b * a.Hq + h) * a.S + split;
      a.part_o[pi * D + d] = acc;
      if (d == 0) {
        a.part_ml[2 * pi] = mm;
        a.part_ml[2 * pi + 1] = lsum;
      }
    }
  }

  if (COUNT && !FINE && lane == 0) {
#pragma unroll
    for (int g = 0; g < CNG; ++g)
#pragma unroll
      for (int c = 0; c < 3; ++c)
        if (cnt[g][c]) atomicAdd(&a.counters[3 * g + c], (unsigned long long)cnt[g][c]);
    if (cnt_vis) atomicAdd(&a.counters[3 * NG], (unsigned long long)cnt_vis);
  }
  if constexpr (COUNT && FINE) {
    // every block was counted before the merge barriers; thread g turns the
    // split histograms into group g's counts
    if (tid < NG) {
      unsigned int skip = 0, full = 0, vis = 0;
      for (int v = 0; v <= NG; ++v) {
        const unsigned int hl = s_hist[v], hr = s_hist[NG + 1 + v];
        vis += hl;
        skip += (v > tid) ? hl : 0u;
        full += (v <= tid) ? hr : 0u;
      }
      if (skip) atomicAdd(&a.counters[3 * tid], (unsigned long long)skip);
      if (vis - skip - full) atomicAdd(&a.counters[3 * tid + 1], (unsigned long long)(vis - skip - full));
      if (full) atomicAdd(&a.counters[3 * tid + 2], (unsigned long long)full);
      if (tid == 0 && vis) atomicAdd(&a.counters[3 * NG], (unsigned long long)vis);
    }
  }
}

// One wave per (sequence, query head of this launch): O = sum_s 2^(m_s - m*)
// o_s / sum_s 2^(m_s - m*) l_s.
template <int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecodeArgs a) {
  const int bh = blockIdx.x;
  const int b = bh / a.Hq;
  const int h = bh - b * a.Hq;
  const int kvh = h / a.r;
  const int ho = kvh * a.rs + (h - kvh * a.r);    // the head's index among the model's heads
  const int lane = threadIdx.x;
  const int64_t base = (int64_t)bh * a.S;
  float mm = -INFINITY;
  for (int s = 0; s < a.S; ++s) mm = fmaxf(mm, a.part_ml[2 * (base + s)]);
  constexpr int PER = D / 64;
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  float lsum = 0.f;
  if (mm != -INFINITY) {
    for (int s = 0; s < a.S; ++s) {
      const float ms = a.part_ml[2 * (base + s)];
      const float sc = (ms == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ms - mm);
      lsum += sc * a.part_ml[2 * (base + s) + 1];
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] += sc * a.part_o[(base + s) * D + lane + 64 * e];
    }
  }
  const float inv = (lsum > 0.f) ? 1.f / lsum : 0.f;
  bf16* op = a.o + (int64_t)b * a.os_b + (int64_t)ho * a.os_h;
#pragma unroll
  for (int e = 0; e < PER; ++e) op[lane + 64 * e] = static_cast<__bf16>(acc[e] * inv);
}

template <int D, int G, bool COMPACT, int HS>
hipError_t launch_dgh(const DecodeArgs& a, bool count, hipStream_t s) {
  const long long blocks = (long long)a.B * a.Hkv * a.S;
  if (blocks <= 0) return hipSuccess;
  if (count)
    hipLaunchKernelGGL((decode_split_kernel<D, G, true, COMPACT, HS>), dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((decode_split_kernel<D, G, false, COMPACT, HS>), dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3((unsigned)(a.B * a.Hq)), dim3(64), 0, s, a);
  return hipGetLastError();
}

// one head set for up to 16 query heads per kv head, two for up to 32
template <int D, int G, bool COMPACT>
hipError_t launch_dg(const DecodeArgs& a, bool count, hipStream_t s) {
  return a.r > 16 ? launch_dgh<D, G, COMPACT, 2>(a, count, s) : launch_dgh<D, G, COMPACT, 1>(a, count, s);
}

template <int D, int G>
hipError_t launch_dgc(const DecodeArgs& a, bool count, hipStream_t s) {
  return a.compact ? launch_dg<D, G, true>(a, count, s) : launch_dg<D, G, false>(a, count, s);
}

// One thread per 16-byte chunk of a key row: the chunk's group g sends it
// to slot (pos0[b] + t) % kcap[g] of that group's ring.  Tokens that a later
// token of the same call would overwrite (t < T - kcap[g]) are skipped, so
// the result does not depend on the order of the writes.
__global__ __launch_bounds__(256) void kcache_append_kernel(KAppendArgs a) {
  const int cpr = a.d_h / 8;                               // chunks per row
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long total = (long long)a.B * a.T * a.Hkv * cpr;
  if (idx >= total) return;
  const int c = (int)(idx % cpr);
  long long r = idx / cpr;
  const int h = (int)(r % a.Hkv);
  r /= a.Hkv;
  const int t = (int)(r % a.T);
  const int b = (int)(r / a.T);
  const int g = (8 * c) / a.G;
  const int cap = a.kcap[g];
  if (t < a.T - cap) return;
  const long long pos = (long long)a.pos0[b] + t;
  if (pos < 0) return;
  const int slot = (int)(pos % cap);
  const u32x4 v = *reinterpret_cast<const u32x4*>(a.k + (int64_t)b * a.ks_b + (int64_t)t * a.ks_t +
                                                   (int64_t)h * a.ks_h + 8 * c);
  bf16* dst = a.store + (int64_t)b * a.ss_b + (int64_t)h * a.ss_h + a.koff[g] + (int64_t)slot * a.G +
              (8 * c) % a.G;
  *reinterpret_cast<u32x4*>(dst) = v;
}

}  // namespace

// Partial results of the decode entry point that allocates nothing: one
// file-scope array per GPU, held until the process ends.  Host code never
// passes the array's name to a kernel (on the host it is only a stand-in
// for the symbol); it uses the device address from hipGetSymbolAddress.
static __device__ __attribute__((aligned(256))) unsigned char scratch[kDecodeScratchBytes];

hipError_t decode_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    // with this device current: its own copy of the array, at its own address
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_decode(const DecodeArgs& a, int d_h, int G, bool count, hipStream_t s) {
  if (d_h == 128 && G == 16) return launch_dgc<128, 16>(a, count, s);
  if (d_h == 128 && G == 32) return launch_dgc<128, 32>(a, count, s);
  if (d_h == 64 && G == 16) return launch_dgc<64, 16>(a, count, s);
  if (d_h == 64 && G == 32) return launch_dgc<64, 32>(a, count, s);
  // fine groups: the full K cache only
  if (a.compact) return hipErrorInvalidValue;
  if (d_h == 128 && G == 8) return launch_dg<128, 8, false>(a, count, s);
  if (d_h == 128 && G == 4) return launch_dg<128, 4, false>(a, count, s);
  if (d_h == 128 && G == 2) return launch_dg<128, 2, false>(a, count, s);
  if (d_h == 64 && G == 8) return launch_dg<64, 8, false>(a, count, s);
  if (d_h == 64 && G == 4) return launch_dg<64, 4, false>(a, count, s);
  if (d_h == 64 && G == 2) return launch_dg<64, 2, false>(a, count, s);
  return hipErrorInvalidValue;
}

hipError_t launch_kcache_append(const KAppendArgs& a, hipStream_t s) {
  const long long total = (long long)a.B * a.T * a.Hkv * (a.d_h / 8);
  if (total <= 0) return hipSuccess;
  const long long blocks = (total + 255) / 256;
  hipLaunchKernelGGL(kcache_append_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace wp
