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
//  * A workgroup is 8 waves (2 per SIMD, one workgroup per CU) that share
//    one kv head and one key range: with GQA ratio >= 4 the waves are 4
//    query heads x 2 blocks of 32 queries, so every K/V tile staged in LDS
//    feeds 256 query rows.  Waves of one query block have identical tile
//    classes.
//  * K and V tiles go from HBM straight into LDS (buffer_load_dwordx4 ...
//    lds: no register staging, rows past the sequence end arrive as zeros).
//    The buffer resources of a tile start at its first key and end after its
//    last, so every offset is within one tile (32-bit, whatever the length).
//    Both are stored row-major with an XOR swizzle of their 16-byte chunks.
//    LDS has 64 banks of 4 bytes (one 256-byte bank row) and serves 16 lanes
//    of a 16-byte read at a time, so K is swizzled by the index of the row's
//    bank row (row for d_h = 128, row / 2 for d_h = 64): the MFMA operand
//    reads of 16 consecutive rows then hit all 64 banks once.  V is swizzled
//    by (row & 3), so the transposing reads (ds_read_b64_tr_b16) of 4 rows
//    hit distinct banks.  A V^T operand of
//    the P.V MFMA is two transposing reads: each returns, to a lane, 4
//    consecutive keys at one head dim -- exactly the two runs of 4 keys
//    that the lane's S^T registers hold.  Two LDS stages: tile t+1 streams
//    in while tile t is consumed; one barrier per tile.
//  * The running max is refreshed (and O rescaled) only when it grows by more
//    than 8 in log2 units, so every probability stays below 2^8; the final
//    O / l and the LSE are unaffected.
//  * Workgroups run heaviest (last query blocks) first; kv head is the
//    fastest-varying block index so that on 8 kv heads each XCD (blocks are
//    dealt round-robin to the 8 XCDs) keeps one kv head's K/V in its L2.
#include "wp_device.h"
#include "wp_internal.h"

namespace wp {

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = 8;
constexpr int kTileKeys = 64;     // keys per tile: two 32-key MFMA blocks, one class per group

template <int D, int G, bool COUNT>
__global__ __launch_bounds__(kThreads) void prefill_kernel(PrefillArgs a) {
  constexpr int NCH = D / 16;         // 16-dim MFMA steps
  constexpr bool FINE = G < 16;       // several groups per MFMA step (G = 2: one per channel)
  constexpr int GC = FINE ? 1 : G / 16;   // MFMA steps per group (coarse groups)
  constexpr int NG = D / G;           // groups
  constexpr int ND = D / 32;          // 32-dim output blocks
  constexpr int RB = D * 2;           // bytes per K/V row in LDS (no padding)
  constexpr int CPR = D / 8;          // 16-byte chunks per row
  constexpr int TILE_B = kTileKeys * RB;                 // bytes per K (or V) tile
  constexpr int LOADS = TILE_B / (kWaves * 64 * 16);     // DMA loads per wave per tile
  constexpr int VX = CPR / 4;          // V swizzle unit: chunk ^= (row & 3) * VX
  constexpr int KRB = 256 / RB;        // K rows per 256-byte LDS bank row
  static_assert(LOADS >= 1 && (TILE_B % (kWaves * 64 * 16)) == 0, "tile shape");

  // LDS: [stage][K tile | V tile]; tile t is read from stage t&1 while tile
  // t+1 streams into the other stage
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2][2 * TILE_B];

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
  const int krow_b = (int)(a.ks_t * 2);     // bytes between consecutive keys in HBM
  const int vrow_b = (int)(a.vs_t * 2);

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

  // ---- DMA of one tile into LDS.  Load i of this wave fills LDS chunks
  //      p = (wave*LOADS + i)*64 + lane (16 bytes each); chunk p holds row
  //      p / CPR, logical chunk (p % CPR) ^ swizzle(row). ----
  int koff[LOADS], voff[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int p = (wave * LOADS + i) * 64 + lane;
    const int row = p / CPR;
    const int pc = p % CPR;
    koff[i] = row * krow_b + (pc ^ ((row / KRB) & (CPR - 1))) * 16;
    voff[i] = row * vrow_b + (pc ^ ((row & 3) * VX)) * 16;
  }
  // each tile's buffer resources start at its first key and span its own
  // rows (at most 64), so offsets stay 32-bit whatever the sequence length
  auto load_tile = [&](int j0, int stage) {
    const int rows = min(kTileKeys, n - j0);                  // >= 1
    const __amdgpu_buffer_rsrc_t kr =
        uniform_rsrc(kbase + (int64_t)j0 * a.ks_t, (rows - 1) * krow_b + 2 * D);
    const __amdgpu_buffer_rsrc_t vr =
        uniform_rsrc(vbase + (int64_t)j0 * a.vs_t, (rows - 1) * vrow_b + 2 * D);
    unsigned char* kdst = &smem[stage][0];
    unsigned char* vdst = &smem[stage][TILE_B];
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int dst = (wave * LOADS + i) * 1024;
      dma16(kr, kdst + dst, koff[i]);
      dma16(vr, vdst + dst, voff[i]);
    }
  };

  // ---- per-lane LDS read offsets (bytes, relative to a stage) ----
  // K operand of S^T: lane reads row 32kb + l32, logical chunk 2s + hh of
  // MFMA step s; physical chunk (2s + hh) ^ swizzle(l32) (the swizzle of
  // rows 32kb + l32 does not depend on kb).
  const int xk = (l32 / KRB) & (CPR - 1);
  int kread[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) kread[c] = l32 * RB + ((2 * c + hh) ^ xk) * 16;
  // V^T operand of P.V via two transposing reads.  In a 16-lane group, lane
  // j = 4e + q reads 4 dims [D0 + 4q, D0 + 4q + 4) of key row K0 + e; lane i
  // then holds keys K0..K0+3 at dim D0 + i.  Here D0 = 32db + 16*(group&1),
  // K0 = 16kc + 4hh (+ 8 for the second read).
  const int grp = lane >> 4;
  const int e4 = (lane & 15) >> 2;
  const int q4 = lane & 3;
  int vread[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db) {
    const int chunk = 4 * db + 2 * (grp & 1) + (q4 >> 1);
    vread[db] = (4 * hh + e4) * RB + (chunk ^ (e4 * VX)) * 16 + (q4 & 1) * 8;
  }

  float m_i = -INFINITY;   // running max (log2 domain), possibly stale by < 8
  float l_i = 0.f;         // running sum (this lane's half of the keys)
  f32x16 o[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;

  // Tile-class counters.  Coarse groups: per-group counts in registers.
  // Fine groups (up to 64): a workgroup histogram of splitL and splitR in
  // LDS, turned into per-group counts at the end (group g is skipped on a
  // tile with splitL > g and full on one with splitR <= g).
  constexpr int CNG = FINE ? 1 : NG;
  unsigned int cnt[CNG][3];
  unsigned int cnt_vis = 0;
  __shared__ unsigned int s_hist[(COUNT && FINE) ? 2 * (NG + 1) : 1];
  if (COUNT) {
#pragma unroll
    for (int g = 0; g < CNG; ++g) cnt[g][0] = cnt[g][1] = cnt[g][2] = 0;
    if (FINE && tid < 2 * (NG + 1)) s_hist[tid] = 0;
  }

  const float sl2 = a.scale_log2;
  const f32x16 zero16 = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};

  // Fine groups (up to 64): the cutoff table in LDS, and split points
  // carried from tile to tile.  A wave meets its key tiles in ascending
  // order, so the tile distances, and with them splitL and splitR, only
  // decrease; a few table reads per tile replace a 2 x 64-step scan.
  // cL / cR hold the cutoff of group fL - 1 / fR - 1 in scalar registers,
  // so a tile whose split points do not move reads no LDS.
  __shared__ int s_cut[FINE ? NG : 1];
  int fL = NG, fR = NG;
  int cL = 0, cR = 0;
  if constexpr (FINE) {
    if (tid < NG) s_cut[tid] = a.cut[tid];
  }
  auto cut_at = [&](int g) { return __builtin_amdgcn_readfirstlane(s_cut[g]); };

  load_tile(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if constexpr (FINE) cL = cR = cut_at(NG - 1);

  for (int it = 0; it < nk; ++it) {
    const int j0 = it * kTileKeys;
    const int stage = it & 1;
    if (it + 1 < nk) load_tile(j0 + kTileKeys, stage ^ 1);
    const unsigned char* sk = &smem[stage][0];
    const unsigned char* sv = &smem[stage][TILE_B];
    if (wave_valid && j0 <= i1w) {
      // ---- classify the (32 queries x 64 keys) tile ----
      const int j1 = min(n - 1, j0 + kTileKeys - 1);
      const int lD = max(0, i0w - j1);
      const int rD = i1w - j0;
      // cutoffs are non-decreasing: splitL / splitR = 1 + last group below
      int sL = 0, sR = 0;
      if constexpr (FINE) {
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
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          sL = (a.cut[g] < lD) ? g + 1 : sL;
          sR = (a.cut[g] < rD) ? g + 1 : sR;
        }
        sL = __builtin_amdgcn_readfirstlane(sL);
        sR = __builtin_amdgcn_readfirstlane(sR);
      }
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

      // K operand of MFMA step c for key block kb
      auto kop = [&](int kb, int c) {
        return *reinterpret_cast<const u32x4*>(sk + kb * 32 * RB + kread[c]);
      };

      // ---- S^T = K Q^T: full groups [sR, NG) as one chain of MFMA steps
      //      from the highest down to step sR * GC.  The K operands of step
      //      c-1 are read right after the MFMAs of step c are issued, so the
      //      LDS latency overlaps their execution. ----
      f32x16 s0 = zero16, s1 = zero16;
      // first MFMA step whose groups are all full
      const int c_end = FINE ? (sR * G + 15) / 16 : sR * GC;
      if (c_end < NCH) {
        const unsigned skb = lds_addr(sk);
        u32x4 ka0, ka1;
        k_reads<32 * RB>(ka0, ka1, skb + kread[NCH - 1]);
#pragma unroll
        for (int cc = NCH - 1; cc >= 0; --cc) {
          s0 = mfma32(ka0, qr[cc], cc == NCH - 1 ? zero16 : s0);
          s1 = mfma32(ka1, qr[cc], cc == NCH - 1 ? zero16 : s1);
          if (cc == c_end) break;
          __builtin_amdgcn_sched_barrier(0);
          k_reads<32 * RB>(ka0, ka1, skb + kread[cc - 1]);
        }
      }

      if constexpr (FINE) {
        // ---- steps [sL*G/16, c_end) mix classes: their full groups join S
        //      with the other words of the operand zeroed, each partial
        //      group gets its own masked MFMA ----
        const int c_lo = (sL * G) / 16;
        if (c_lo < c_end) {
          const int base = (i0w + l32) - j0;     // dist = base - (32kb + out_row(r))
#pragma unroll
          for (int c = 0; c < NCH; ++c) {
            if (c < c_lo || c >= c_end) continue;
            const u32x4 k0 = kop(0, c), k1 = kop(1, c);
            // group of operand word w (head dims 16c + 8hh + 2w, +1)
            auto grp = [&](int w) { return (16 * c + 8 * hh + 2 * w) / G; };
            if ((16 * c + 15) / G >= sR) {
              s0 = mfma32(keep_words(k0, [&](int w) { return grp(w) >= sR; }), qr[c], s0);
              s1 = mfma32(keep_words(k1, [&](int w) { return grp(w) >= sR; }), qr[c], s1);
            }
            // a runtime loop over just this step's partial groups (unrolled
            // over all 16/G groups of every step, the code outgrows the
            // instruction cache)
#pragma unroll 1
            for (int g = max((16 * c) / G, sL); g < min((16 * c + 15) / G + 1, sR); ++g) {
              const int cg = cut_at(g);
              f32x16 t = mfma32(keep_words(k0, [&](int w) { return grp(w) == g; }), qr[c], zero16);
#pragma unroll
              for (int r = 0; r < 16; ++r) s0[r] += (base - out_row(r, hh) <= cg) ? t[r] : 0.f;
              t = mfma32(keep_words(k1, [&](int w) { return grp(w) == g; }), qr[c], zero16);
#pragma unroll
              for (int r = 0; r < 16; ++r) s1[r] += (base - 32 - out_row(r, hh) <= cg) ? t[r] : 0.f;
            }
          }
        }
      } else if (sL < sR) {
        // ---- partial groups [sL, sR): compute, mask dist <= cutoff, add ----
        const int base = (i0w + l32) - j0;     // dist = base - (32kb + out_row(r))
#pragma unroll
        for (int g = NG - 1; g >= 0; --g) {
          if (g >= sR || g < sL) continue;
          const int cg = a.cut[g];
          f32x16 t = zero16;
#pragma unroll
          for (int c = 0; c < GC; ++c) t = mfma32(kop(0, g * GC + c), qr[g * GC + c], t);
#pragma unroll
          for (int r = 0; r < 16; ++r) s0[r] += (base - out_row(r, hh) <= cg) ? t[r] : 0.f;
          t = zero16;
#pragma unroll
          for (int c = 0; c < GC; ++c) t = mfma32(kop(1, g * GC + c), qr[g * GC + c], t);
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

      // ---- O^T += V^T P^T; the V^T operand is two transposing reads ----
#pragma unroll
      for (int kc = 0; kc < 4; ++kc)
#pragma unroll
        for (int db = 0; db < ND; ++db) {
          const unsigned char* va = sv + kc * 16 * RB + vread[db];
          const u32x2 lo2 = read_tr16(va);
          const u32x2 hi2 = read_tr16(va + 8 * RB);
          const u32x4 vop = {lo2[0], lo2[1], hi2[0], hi2[1]};
          o[db] = mfma32(vop, p[kc], o[db]);
        }
    }

    // tile it+1 must be in LDS, and every wave done with stage it&1, before
    // the next iteration
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
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
    if (COUNT && !FINE && lane == 0) {
#pragma unroll
      for (int g = 0; g < CNG; ++g)
#pragma unroll
        for (int c = 0; c < 3; ++c)
          if (cnt[g][c]) atomicAdd(&a.counters[3 * g + c], (unsigned long long)cnt[g][c]);
      if (cnt_vis) atomicAdd(&a.counters[3 * NG], (unsigned long long)cnt_vis);
    }
  }
  if constexpr (COUNT && FINE) {
    // every tile was counted before the last barrier of the loop; thread g
    // turns the split histograms into group g's counts
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

template <int D, int G>
hipError_t launch_dg(const PrefillArgs& a0, bool count, hipStream_t s) {
  // each wave takes 32 queries of one head: HPW heads x QSUB query blocks
  PrefillArgs a = a0;
  a.QSUB = kWaves / a.HPW;
  a.QB = 32 * a.QSUB;
  a.nqb = (a.n + a.QB - 1) / a.QB;
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
  if (d_h == 128 && G == 8) return launch_dg<128, 8>(a, count, s);
  if (d_h == 128 && G == 4) return launch_dg<128, 4>(a, count, s);
  if (d_h == 128 && G == 2) return launch_dg<128, 2>(a, count, s);
  if (d_h == 64 && G == 8) return launch_dg<64, 8>(a, count, s);
  if (d_h == 64 && G == 4) return launch_dg<64, 4>(a, count, s);
  if (d_h == 64 && G == 2) return launch_dg<64, 2>(a, count, s);
  return hipErrorInvalidValue;
}

}  // namespace wp
