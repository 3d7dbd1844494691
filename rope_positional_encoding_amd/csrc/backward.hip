// WavePrune causal attention, backward pass, for gfx950.
//
// Gradients of <dO, O> through O = softmax(S) V with the grouped rule
// S_ij = (1/sqrt(d_h)) sum_g [i - j <= D'_g] q_i,g . k_j,g (WavePrune
// reading notes on cc.laoqi.cc, section 2.1, Eq. (6), grouped by section 2.3,
// Eq. (8)).  The same page's kernel paragraph (its summary of the paper's
// Appendix C) describes the backward: the head dimension becomes an output
// axis, so the gradient operands are masked per group before the matrix
// product, and dQ and dK share one mask.  With P = exp(S - LSE) (LSE from the
// forward pass) and Dsum_i = dO_i . O_i:
//   dV_j = sum_i P_ij dO_i,   dP_ij = dO_i . V_j,   dS_ij = P_ij (dP_ij - Dsum_i),
//   dQ_i,g = scale sum_j [i-j <= D'_g] dS_ij k_j,g,
//   dK_j,g = scale sum_i [i-j <= D'_g] dS_ij q_i,g   (and dK, dV summed over
//   the query heads of a kv head).
// Every tile is classified per group as in the forward pass; a skipped group
// contributes to neither dQ nor dK, a full group uses dS as it is, a partial
// group uses dS masked by distance <= cutoff.
//
// gfx950 design:
//  * Three kernels: row sums Dsum (HBM-bound), a dK/dV kernel whose waves
//    each own 32 keys and stream the query tiles of every head of their kv
//    head, and a dQ kernel whose waves each own 32 queries of one head and
//    stream the key tiles.  No atomics: every output element has one writer.
//  * All products run on v_mfma_f32_32x32x16_bf16.  In the dK/dV kernel the
//    logits are computed as S = Q K^T (the lane owns one key column), so P
//    and dS are already the B operands of dV^T = dO^T P and dK^T = Q^T dS; in
//    the dQ kernel as S^T = K Q^T (the lane owns one query column), so dS^T
//    is the B operand of dQ^T = K^T dS^T.  The transposed A operands (dO^T,
//    Q^T, K^T) come from transposing LDS reads (ds_read_b64_tr_b16) of
//    row-major tiles, exactly as V^T in the forward pass.
//  * A tile read both row-wise (16-byte operand reads of 16 rows) and
//    transposed (transposing reads of 4 rows x 4 chunks) gets one XOR
//    swizzle of its 16-byte chunks that keeps both read patterns free of
//    bank conflicts (dual_swz below).
//  * Group masks of the dK^T / dQ^T products: a 32-row output block covers
//    one or two groups (G = 32 / 16).  When they are all full the block takes
//    one MFMA per 16-row k step; otherwise each non-skipped group takes its
//    own MFMA with the A rows of the other group zeroed and its own (masked)
//    dS operand.
//  * Fine groups (G = 2, 4, 8; G = 2 is the exact per-channel rule): a
//    16-dim MFMA step of the logits holds several groups, so the steps that
//    mix classes take their full groups with the other operand words zeroed
//    and each partial group in a masked MFMA of its own; a 32-row block of
//    dK^T / dQ^T takes its full groups in one MFMA set and its partial groups
//    in a run-time loop (unrolled over up to 16 groups per block, the code
//    would outgrow the instruction cache).
#include "wp_device.h"
#include "wp_internal.h"

namespace wp {

namespace {

// XOR swizzle of the 16-byte chunks of tile row `row` (bijective on the
// chunks of a row).  Row-wise reads: 16 lanes read rows R..R+15 at one
// logical chunk; with 256-byte rows (d_h = 128) every row covers all 64 banks
// and the swizzle must give the 16 rows distinct chunks; with 128-byte rows
// two rows share a bank row and the 8 rows of one parity must differ.
// Transposing reads: 32 lanes read rows R0..R0+3 (R0 % 4 == 0) at logical
// chunks 4m..4m+3, which must land on 16 distinct chunk positions.
template <int D>
__device__ inline int dual_swz(int row) {
  if constexpr (D == 128)
    return ((row & 3) << 2) | ((row >> 2) & 3);
  else
    return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

__device__ inline float bf16_lo(unsigned int w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(unsigned int w) { return __uint_as_float(w & 0xffff0000u); }

// Row values of query i of head h: its LSE in base 2 and Dsum[b][h][i] =
// sum_d dO[b,i,h,d] * O[b,i,h,d] (float32, bf16 inputs), stored as a pair.
template <int D>
__global__ __launch_bounds__(256) void bwd_dsum_kernel(BackwardArgs a) {
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long rows = (long long)a.B * a.n * a.Hq;
  if (idx >= rows) return;
  const int h = (int)(idx % a.Hq);
  const long long bi = idx / a.Hq;
  const int i = (int)(bi % a.n);
  const int b = (int)(bi / a.n);
  const bf16* op = a.o + (int64_t)b * a.os_b + (int64_t)i * a.os_t + (int64_t)h * a.os_h;
  const bf16* gp = a.dout + (int64_t)b * a.gs_b + (int64_t)i * a.gs_t + (int64_t)h * a.gs_h;
  float acc = 0.f;
#pragma unroll
  for (int c = 0; c < D / 8; ++c) {
    const u32x4 x = *reinterpret_cast<const u32x4*>(op + 8 * c);
    const u32x4 y = *reinterpret_cast<const u32x4*>(gp + 8 * c);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc = __builtin_fmaf(bf16_lo(x[w]), bf16_lo(y[w]), acc);
      acc = __builtin_fmaf(bf16_hi(x[w]), bf16_hi(y[w]), acc);
    }
  }
  const int64_t r = ((int64_t)b * a.Hq + h) * a.n + i;
  *reinterpret_cast<float2*>(a.rowv + 2 * r) = float2{a.lse[r] * 1.4426950408889634f, acc};
}

// Classes of a tile from its causal distance range [lD, rD]: groups [0, sL)
// skip, [sL, sR) partial, [sR, NG) full (cutoffs non-decreasing).
template <int NG>
__device__ inline void split_points(const int* cut, int lD, int rD, int& sL, int& sR) {
  sL = 0;
  sR = 0;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    sL = (cut[g] < lD) ? g + 1 : sL;
    sR = (cut[g] < rD) ? g + 1 : sR;
  }
  sL = __builtin_amdgcn_readfirstlane(sL);
  sR = __builtin_amdgcn_readfirstlane(sR);
}

// Packs a 32x32 output block (this lane's 16 values) into the two B operands
// of the 16-row k steps that follow (rows 0..15 -> [0], 16..31 -> [1]), in
// the order the transposing A reads deliver their rows.
__device__ inline void pack_block(const f32x16& x, u32x4 (&p)[2]) {
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int w = 0; w < 4; ++w) p[c][w] = pack_bf16x2(x[8 * c + 2 * w], x[8 * c + 2 * w + 1]);
}

// Zeroes the bf16 entries of a packed block (pack_block's layout) whose
// row r fails keep(r): word p[c][w] holds rows 8c + 2w (low half) and
// 8c + 2w + 1 (high half) of this lane's 16 values.
template <typename F>
__device__ inline void mask_block(u32x4 (&p)[2], F keep) {
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const unsigned lo = keep(8 * c + 2 * w) ? 0x0000ffffu : 0u;
      const unsigned hi = keep(8 * c + 2 * w + 1) ? 0xffff0000u : 0u;
      p[c][w] &= lo | hi;
    }
}

// ---------------------------------------------------------------------------
// dK / dV.  A workgroup owns 128 keys of one kv head and streams the 32-query
// tiles of every query head of that kv head.  Its 8 waves work in pairs;
// pair p owns keys keyw + 32p .. +31:
//  * wave p (K^T resident) forms S = Q K^T and P for tile u, hands P to its
//    partner through LDS and accumulates dV^T += dO^T P;
//  * wave 4 + p (V^T resident) takes tile u one step later: dP = dO V^T,
//    dS = P (dP - Dsum), dK^T += Q^T dS.
// Each wave then holds one 32x128 accumulator and one resident operand,
// which keeps it under 256 registers: the two waves of a SIMD overlap one's
// exponentials with the other's MFMAs.  Tiles (Q, dO and the rows' LSE and
// Dsum) arrive by DMA kPrefetch steps ahead of the first waves' use.
// ---------------------------------------------------------------------------
constexpr int kKvWaves = 8;
constexpr int kKvThreads = 64 * kKvWaves;
constexpr int kPrefetch = 2;                      // tiles in flight ahead of use
constexpr int kStages = kPrefetch + 2;            // + the tiles of both halves of a pair

// compile-time role of a wave in a pair (the two roles run separate loops,
// so that each loop updates its accumulators along one code path)
template <bool P>
struct Role {
  static constexpr bool first = P;
};

template <int N>
__device__ inline void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(N) : "memory");
}
// Barrier without the fence of __syncthreads, which would wait for every DMA
// in flight; callers wait for what they need first.
__device__ inline void bare_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int D, int G>
__global__ __launch_bounds__(kKvThreads) void bwd_dkdv_kernel(BackwardArgs a) {
  constexpr int NCH = D / 16;
  constexpr bool FINE = G < 16;                   // several groups per 16-dim MFMA step
  constexpr int GC = FINE ? 1 : G / 16;
  constexpr int NG = D / G;
  constexpr int ND = D / 32;
  constexpr int RB = D * 2;
  constexpr int CPR = D / 8;
  constexpr int TILE_B = 32 * RB;                           // one 32-row tile
  constexpr int TCH = TILE_B / 16;                          // its 16-byte chunks
  constexpr int NL = 2 * TCH / kKvThreads;                  // DMA loads per lane and tile
  static_assert(NL >= 1 && (2 * TCH) % kKvThreads == 0 && TCH % 64 == 0, "tile shape");

  // [stage][Q tile | dO tile]; the rows' (log2 LSE, Dsum) pairs per stage;
  // P of each pair, float, [parity][pair][r / 4][lane][r % 4]
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kStages][2 * TILE_B];
  __shared__ __attribute__((aligned(256))) float s_ld[kStages][64];
  __shared__ __attribute__((aligned(16))) float s_p[2][4][16 * 64];
  // fine groups: the cutoff table, read with wave-uniform indexes
  __shared__ int s_cut[FINE ? NG : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pair = wave & 3;
  if constexpr (FINE) {
    if (tid < NG) s_cut[tid] = a.cut[tid];
  }
  auto cut_at = [&](int g) { return __builtin_amdgcn_readfirstlane(s_cut[g]); };
  // fine groups: split points carried from tile to tile.  Within one query
  // head a wave meets its query tiles in ascending order, so the distances
  // and the split points only grow; they restart at the head's first tile.
  int fL = 0, fR = 0;
  const bool pwave = wave < 4;                     // forms P and dV (else dP, dS, dK)
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  // block decomposition, kept scalar (the divisions run on the vector unit)
  int bid = blockIdx.x;
  const int kvh = __builtin_amdgcn_readfirstlane(bid % a.Hkv);
  bid /= a.Hkv;
  const int b = __builtin_amdgcn_readfirstlane(bid % a.B);
  const int kblk = __builtin_amdgcn_readfirstlane(bid / a.B);   // ascending: most query tiles first
  const int n = a.n;
  const int keyw = kblk * 128;                     // first key of the workgroup
  const int key0 = __builtin_amdgcn_readfirstlane(keyw + 32 * pair);
  const int key1 = __builtin_amdgcn_readfirstlane(min(n, key0 + 32) - 1);
  const bool wave_valid = key0 < n;

  // the resident B operand, K^T or V^T: lane owns key key0 + l32, dims
  // [16c + 8hh, +8) of step c
  u32x4 br[NCH];
  {
    const int j = key0 + l32;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    const bf16* p = pwave ? a.k + (int64_t)b * a.ks_b + (int64_t)j * a.ks_t + (int64_t)kvh * a.ks_h
                          : a.v + (int64_t)b * a.vs_b + (int64_t)j * a.vs_t + (int64_t)kvh * a.vs_h;
    p += hh * 8;
#pragma unroll
    for (int c = 0; c < NCH; ++c) br[c] = (j < n) ? *reinterpret_cast<const u32x4*>(p + c * 16) : zero;
  }

  // DMA: load i of an issuing lane fills chunk p of a stage ([Q | dO], TCH
  // chunks each): tile row pt / CPR, logical chunk (pt % CPR) ^
  // dual_swz(row), pt = p % TCH.  Coarse groups: only the first waves issue
  // it, p = wave*64 + lane + 256*i (2 NL loads per lane): the second waves
  // set the pace of a step and the first waves wait for them at the barrier
  // anyway (10% faster at 32K, G = 16).  Fine groups keep the first waves
  // busier with their per-group loops, so all eight waves share the DMA
  // there, p = wave*64 + lane + 512*i.
  const int qrow_b = (int)(a.qs_t * 2);
  const int grow_b = (int)(a.gs_t * 2);
  constexpr bool DMA1 = !FINE;                  // DMA by the first waves only
  constexpr int NLD = DMA1 ? 2 * NL : NL;       // DMA loads per issuing lane and tile
  constexpr int DSTRIDE = DMA1 ? 256 : kKvThreads;
  int doff[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int p = (DMA1 ? (wave & 3) : wave) * 64 + lane + DSTRIDE * i;
    const int pt = p % TCH;
    const int row = pt / CPR;
    doff[i] = row * (p < TCH ? qrow_b : grow_b) + ((pt % CPR) ^ dual_swz<D>(row)) * 16;
  }
  // Tiles t = 0 .. total-1: head hr = t / nt of this kv head, queries from
  // (t0 + ti) * 32, ti = t % nt.  Head and tile index are stepped as scalar
  // counters (an integer division would run on the vector unit).
  const int t0 = keyw / 32;
  const int nt = __builtin_amdgcn_readfirstlane((n + 31) / 32 - t0);   // >= 1 (keyw < n)
  const int total = a.r * nt;
  // tile (hr, ti): its Q / dO rows go to dst, its 32 row pairs to ldst
  // (wave 0, lanes 0-15, 16 bytes each; rows past the end read as zero and
  // are masked)
  auto load_tile = [&](int hr, int ti, unsigned char* dst, float* ldst) {
    const int h = kvh * a.r + hr;
    const int i0 = (t0 + ti) * 32;
    const int rows = min(32, n - i0);         // the tile's own rows: 32-bit offsets
    const __amdgpu_buffer_rsrc_t qrs = uniform_rsrc(
        a.q + (int64_t)b * a.qs_b + (int64_t)i0 * a.qs_t + (int64_t)h * a.qs_h, (rows - 1) * qrow_b + 2 * D);
    const __amdgpu_buffer_rsrc_t grs = uniform_rsrc(
        a.dout + (int64_t)b * a.gs_b + (int64_t)i0 * a.gs_t + (int64_t)h * a.gs_h, (rows - 1) * grow_b + 2 * D);
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int p0 = wave * 64 + DSTRIDE * i;  // wave-uniform: Q or dO
      dma16(p0 < TCH ? qrs : grs, dst + p0 * 16, doff[i]);
    }
    if (wave == 0 && lane < 16)
      dma16(uniform_rsrc(a.rowv + 2 * (((int64_t)b * a.Hq + h) * n + i0), min(rows, 32) * 8), ldst, lane * 16);
  };

  // row-wise A reads (rows l32 of a tile, logical chunk 2c + hh)
  int rread[NCH];
  {
    const int sw = dual_swz<D>(l32);
#pragma unroll
    for (int c = 0; c < NCH; ++c) rread[c] = l32 * RB + ((2 * c + hh) ^ sw) * 16;
  }
  // transposing A reads: rows 16kc + 4hh + e4 (lo) and + 8 (hi), logical
  // chunk 4db + 2(group&1) + (q4>>1), half (q4&1); the swizzle of those
  // rows does not depend on kc
  const int grp = lane >> 4;
  const int e4 = (lane & 15) >> 2;
  const int q4 = lane & 3;
  int tlo[ND], thi[ND];
  {
    const int rlo = 4 * hh + e4, rhi = rlo + 8;
#pragma unroll
    for (int db = 0; db < ND; ++db) {
      const int chunk = 4 * db + 2 * (grp & 1) + (q4 >> 1);
      tlo[db] = rlo * RB + (chunk ^ dual_swz<D>(rlo)) * 16 + (q4 & 1) * 8;
      thi[db] = rhi * RB + (chunk ^ dual_swz<D>(rhi)) * 16 + (q4 & 1) * 8;
    }
  }

  // dV^T (first wave of a pair) or dK^T (second): rows dims, columns keys
  f32x16 acc[ND];
  const f32x16 zero16 = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int db = 0; db < ND; ++db) acc[db] = zero16;
  const float sl2 = a.scale_log2;
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  const int jkey = key0 + l32;                     // this lane's key

  // One step: start the DMA of tile u + kPrefetch into (dst, ldst); the first
  // waves process tile u, the second waves tile u - 1, from (sq, sg, sl) and
  // the P buffer pb.  The restrict-qualified pointers tell the compiler that
  // the step's LDS reads never touch the DMA destination, so it does not
  // hold them until the DMA lands; the waits and barrier after each step
  // order the stages.  (lhr, lti): head and query tile index of the tile to
  // load; cti: query tile index of the tile to process.
  auto step = [&](auto role, int u, int lhr, int lti, int cti, const unsigned char* __restrict__ sq,
                  const unsigned char* __restrict__ sg, const float* __restrict__ sl, float* __restrict__ pb,
                  unsigned char* __restrict__ dst, float* __restrict__ ldst) {
    constexpr bool PW = decltype(role)::first;
    if ((!DMA1 || PW) && u + kPrefetch < total) load_tile(lhr, lti, dst, ldst);
    const int v = PW ? u : u - 1;
    const int i0 = __builtin_amdgcn_readfirstlane((t0 + cti) * 32);
    const int i1 = min(n, i0 + 32) - 1;
    if (FINE && cti == 0) {
      fL = 0;
      fR = 0;
    }
    if (!(v >= 0 && v < total && wave_valid && i1 >= key0)) return;
    const int lD = max(0, i0 - key1);
    const int rD = i1 - key0;
    int sL, sR;
    if constexpr (FINE) {
      while (fL < NG && cut_at(fL) < lD) ++fL;
      while (fR < NG && cut_at(fR) < rD) ++fR;
      sL = fL;
      sR = fR;
    } else {
      split_points<NG>(a.cut, lD, rD, sL, sR);
    }
    auto rop = [&](const unsigned char* t, int c) { return *reinterpret_cast<const u32x4*>(t + rread[c]); };
    if constexpr (PW) {
      // ---- S = Q K^T: full groups [sR, NG) as one chain, then partials ----
      f32x16 s = zero16;
      if constexpr (FINE) {
        // steps [c_end, NCH) hold full groups only: one chain; steps
        // [c_lo, c_end) mix classes: their full groups join with the other
        // dims of the K operand zeroed, each partial group gets its own
        // masked MFMA (a run-time loop over just the step's partial groups)
        const int c_end = (sR * G + 15) / 16;
        const int c_lo = (sL * G) / 16;
        if (c_end < NCH) {
          s = mfma32(rop(sq, NCH - 1), br[NCH - 1], zero16);
#pragma unroll
          for (int cc = NCH - 2; cc >= 0; --cc) {
            if (cc < c_end) break;
            s = mfma32(rop(sq, cc), br[cc], s);
          }
        }
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          if (c < c_lo || c >= c_end) continue;
          const u32x4 qa = rop(sq, c);
          auto grp = [&](int w) { return (16 * c + 8 * hh + 2 * w) / G; };
          if ((16 * c + 15) / G >= sR) s = mfma32(qa, keep_words(br[c], [&](int w) { return grp(w) >= sR; }), s);
#pragma unroll 1
          for (int g = max((16 * c) / G, sL); g < min((16 * c + 15) / G + 1, sR); ++g) {
            const int cg = cut_at(g);
            const f32x16 t = mfma32(qa, keep_words(br[c], [&](int w) { return grp(w) == g; }), zero16);
#pragma unroll
            for (int r = 0; r < 16; ++r) s[r] += (i0 + out_row(r, hh) - jkey <= cg) ? t[r] : 0.f;
          }
        }
      } else {
      if (sR < NG) {
        s = mfma32(rop(sq, NCH - 1), br[NCH - 1], zero16);
#pragma unroll
        for (int cc = NCH - 2; cc >= 0; --cc) {
          if (cc < sR * GC) break;
          s = mfma32(rop(sq, cc), br[cc], s);
        }
      }
      if (sL < sR) {
#pragma unroll
        for (int g = NG - 1; g >= 0; --g) {
          if (g >= sR || g < sL) continue;
          f32x16 t = zero16;
#pragma unroll
          for (int c = 0; c < GC; ++c) t = mfma32(rop(sq, g * GC + c), br[g * GC + c], t);
#pragma unroll
          for (int r = 0; r < 16; ++r) s[r] += (i0 + out_row(r, hh) - jkey <= a.cut[g]) ? t[r] : 0.f;
        }
      }
      }
      // ---- P, to the partner and packed; queries before the key or past
      //      the end are masked, on the tiles that have such queries ----
      f32x16 pm;
      const bool interior = i0 >= key1 && i0 + 31 < n;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int rb = 8 * r4 + 4 * hh;                  // first of 4 consecutive rows
        const float4 x = *reinterpret_cast<const float4*>(sl + 2 * rb);
        const float4 y = *reinterpret_cast<const float4*>(sl + 2 * rb + 4);
        const float lv[4] = {x.x, x.z, y.x, y.z};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          pm[4 * r4 + e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[4 * r4 + e], sl2, -lv[e]));
        if (!interior) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = i0 + rb + e;
            pm[4 * r4 + e] = (i >= jkey && i < n) ? pm[4 * r4 + e] : 0.f;
          }
        }
        *reinterpret_cast<float4*>(pb + (r4 * 64 + lane) * 4) =
            float4{pm[4 * r4], pm[4 * r4 + 1], pm[4 * r4 + 2], pm[4 * r4 + 3]};
      }
      u32x4 pp[2];
      pack_block(pm, pp);
      // ---- dV^T += dO^T P ----
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int db = 0; db < ND; ++db) {
          const u32x2 lo = read_tr16(sg + kc * 16 * RB + tlo[db]);
          const u32x2 hi = read_tr16(sg + kc * 16 * RB + thi[db]);
          acc[db] = mfma32(u32x4{lo[0], lo[1], hi[0], hi[1]}, pp[kc], acc[db]);
        }
    } else {
      // ---- dP = dO V^T ----
      f32x16 dp = mfma32(rop(sg, 0), br[0], zero16);
#pragma unroll
      for (int c = 1; c < NCH; ++c) dp = mfma32(rop(sg, c), br[c], dp);
      // ---- dS = P (dP - Dsum), P from the partner ----
      f32x16 ds;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int rb = 8 * r4 + 4 * hh;
        const float4 x = *reinterpret_cast<const float4*>(sl + 2 * rb);
        const float4 y = *reinterpret_cast<const float4*>(sl + 2 * rb + 4);
        const float dv[4] = {x.y, x.w, y.y, y.w};
        const float4 p4 = *reinterpret_cast<const float4*>(pb + (r4 * 64 + lane) * 4);
        const float pv[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) ds[4 * r4 + e] = pv[e] * (dp[4 * r4 + e] - dv[e]);
      }
      u32x4 dsp[2];
      pack_block(ds, dsp);
      // ---- dK^T += Q^T dS, masked per group.  Each update is a uniform
      //      "if" around in-place MFMAs, so the accumulators stay put. ----
      // full groups [sR, NG): unmasked dS; A rows (dims) of other groups zero
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        const int ga = (32 * db) / G, gb = (32 * db + 31) / G;
        if (gb < sR) continue;                            // no full group in the block
        const u32x2 lo0 = read_tr16(sq + tlo[db]);
        const u32x2 hi0 = read_tr16(sq + thi[db]);
        const u32x2 lo1 = read_tr16(sq + 16 * RB + tlo[db]);
        const u32x2 hi1 = read_tr16(sq + 16 * RB + thi[db]);
        u32x4 a0 = {lo0[0], lo0[1], hi0[0], hi0[1]};
        u32x4 a1 = {lo1[0], lo1[1], hi1[0], hi1[1]};
        if (ga < sR) {
          const bool keep = (32 * db + l32) / G >= sR;
          a0 = keep ? a0 : zero4;
          a1 = keep ? a1 : zero4;
        }
        acc[db] = mfma32(a0, dsp[0], acc[db]);
        acc[db] = mfma32(a1, dsp[1], acc[db]);
      }
      // partial groups [sL, sR): dS masked by the group's cutoff, A rows of
      // the group only
      if constexpr (FINE) {
        // per 32-dim block, a run-time loop over its partial groups
#pragma unroll
        for (int db = 0; db < ND; ++db) {
          const int g_lo = max(sL, (32 * db) / G), g_hi = min(sR, (32 * db + 31) / G + 1);
          if (g_lo >= g_hi) continue;
          const u32x2 lo0 = read_tr16(sq + tlo[db]);
          const u32x2 hi0 = read_tr16(sq + thi[db]);
          const u32x2 lo1 = read_tr16(sq + 16 * RB + tlo[db]);
          const u32x2 hi1 = read_tr16(sq + 16 * RB + thi[db]);
          const u32x4 q0 = {lo0[0], lo0[1], hi0[0], hi0[1]};
          const u32x4 q1 = {lo1[0], lo1[1], hi1[0], hi1[1]};
          const int gl = (32 * db + l32) / G;           // group of this lane's A row
#pragma unroll 1
          for (int g = g_lo; g < g_hi; ++g) {
            u32x4 bop[2] = {dsp[0], dsp[1]};
            const int cg = cut_at(g);
            mask_block(bop, [&](int r) { return i0 + out_row(r, hh) - jkey <= cg; });
            acc[db] = mfma32(gl == g ? q0 : zero4, bop[0], acc[db]);
            acc[db] = mfma32(gl == g ? q1 : zero4, bop[1], acc[db]);
          }
        }
      } else {
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        if (g < sL || g >= sR) continue;
        const int db = (g * G) / 32;
        u32x4 bop[2] = {dsp[0], dsp[1]};
        const int cg = a.cut[g];
        mask_block(bop, [&](int r) { return i0 + out_row(r, hh) - jkey <= cg; });
        const bool mine = ((32 * db + l32) / G) == g;
        const u32x2 lo0 = read_tr16(sq + tlo[db]);
        const u32x2 hi0 = read_tr16(sq + thi[db]);
        const u32x2 lo1 = read_tr16(sq + 16 * RB + tlo[db]);
        const u32x2 hi1 = read_tr16(sq + 16 * RB + thi[db]);
        const u32x4 a0 = mine ? u32x4{lo0[0], lo0[1], hi0[0], hi0[1]} : zero4;
        const u32x4 a1 = mine ? u32x4{lo1[0], lo1[1], hi1[0], hi1[1]} : zero4;
        acc[db] = mfma32(a0, bop[0], acc[db]);
        acc[db] = mfma32(a1, bop[1], acc[db]);
      }
      }
    }
  };

  // The resident operand is complete before the loop (an empty asm use
  // makes the compiler wait for it here, not inside it).
#pragma unroll
  for (int c = 0; c < NCH; ++c) asm volatile("" ::"v"(br[c]));
  // tiles 0 .. kPrefetch-1 into stages 0 .. kPrefetch-1
#pragma unroll
  for (int t = 0; t < kPrefetch; ++t)
    if ((!DMA1 || pwave) && t < total) load_tile(t / nt, t % nt, &smem[t][0], &s_ld[t][0]);
  wait_vm<0>();
  bare_barrier();

  auto run = [&](auto role) {
    constexpr bool PW = decltype(role)::first;
    // (lhr, lti): the next tile to load; cti: the query tile index of the
    // tile this wave processes (-1 before the second waves' first tile)
    int lhr = __builtin_amdgcn_readfirstlane(kPrefetch / nt);
    int lti = __builtin_amdgcn_readfirstlane(kPrefetch % nt);
    int cti = PW ? 0 : -1;
    for (int u = 0; u <= total; ++u) {
      // first waves: tile u; second waves: tile u - 1 (tile t sits in stage
      // t % kStages); the DMA fills the stage of tile u + kPrefetch, last
      // read in step u - 1
      const int v = PW ? u : u - 1;
      const int st = (v + kStages) % kStages;
      const int nx = (u + kPrefetch) % kStages;
      step(role, u, lhr, lti, cti, &smem[st][0], &smem[st][TILE_B], &s_ld[st][0], &s_p[(v + 2) & 1][pair][0],
           &smem[nx][0], &s_ld[nx][0]);
      if (++lti == nt) {
        lti = 0;
        ++lhr;
      }
      if (++cti == nt) cti = 0;
      // tile u + 1 must have landed (later tiles may still be in flight)
      // and every wave be done with this step's stages
      const int ahead = min(total - 1, u + kPrefetch) - (u + 1);   // tiles issued after u + 1
      if (ahead <= 0 || (DMA1 && !PW)) {
        wait_vm<0>();
      } else if (wave == 0) {
        if (ahead == 1) wait_vm<NLD + 1>(); else wait_vm<2 * (NLD + 1)>();
      } else {
        if (ahead == 1) wait_vm<NLD>(); else wait_vm<2 * NLD>();
      }
      bare_barrier();
    }
  };
  if (pwave)
    run(Role<true>{});
  else
    run(Role<false>{});

  // ---- dV = dV^T (first waves), dK = scale * dK^T (second): lane's key,
  // rows = dims ----
  if (wave_valid && jkey < n) {
    const float sc = pwave ? 1.f : a.scale;
    bf16* op = pwave ? a.dv + (int64_t)b * a.dvs_b + (int64_t)jkey * a.dvs_t + (int64_t)kvh * a.dvs_h
                     : a.dk + (int64_t)b * a.dks_b + (int64_t)jkey * a.dks_t + (int64_t)kvh * a.dks_h;
    op += hh * 4;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        u32x2 w;
        w[0] = pack_bf16x2(acc[db][4 * r4] * sc, acc[db][4 * r4 + 1] * sc);
        w[1] = pack_bf16x2(acc[db][4 * r4 + 2] * sc, acc[db][4 * r4 + 3] * sc);
        *reinterpret_cast<u32x2*>(op + db * 32 + r4 * 8) = w;
      }
  }
}

// ---------------------------------------------------------------------------
// dQ: a wave owns 32 queries of one head (4 waves: HPW heads x 4/HPW query
// blocks sharing one kv head); the workgroup streams 64-key K / V tiles.
// ---------------------------------------------------------------------------
constexpr int kDqWaves = 4;
constexpr int kDqThreads = 64 * kDqWaves;

// Two workgroups per CU, except for G = 2 (one cutoff per channel), whose
// per-group loops need more than 256 registers: it runs at one workgroup per
// CU without spilling (measured 4% faster than two with spills; G = 4, 8 are
// faster at two).
template <int D, int G>
__global__ __launch_bounds__(kDqThreads, G == 2 ? 1 : 2) void bwd_dq_kernel(BackwardArgs a) {
  constexpr int NCH = D / 16;
  constexpr bool FINE = G < 16;                   // several groups per 16-dim MFMA step
  constexpr int GC = FINE ? 1 : G / 16;
  constexpr int NG = D / G;
  constexpr int ND = D / 32;
  constexpr int RB = D * 2;
  constexpr int CPR = D / 8;
  constexpr int TILE_B = 64 * RB;
  constexpr int LOADS = TILE_B / (kDqWaves * 64 * 16);
  constexpr int KRB = 256 / RB;
  static_assert(LOADS >= 1 && TILE_B % (kDqWaves * 64 * 16) == 0, "tile shape");

  // [stage][K tile | V tile]
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2][2 * TILE_B];
  // fine groups: the cutoff table, read with wave-uniform indexes
  __shared__ int s_cut[FINE ? NG : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  if constexpr (FINE) {
    if (tid < NG) s_cut[tid] = a.cut[tid];
  }
  auto cut_at = [&](int g) { return __builtin_amdgcn_readfirstlane(s_cut[g]); };
  // fine groups: split points carried from tile to tile (the key tiles come
  // in ascending order, so the distances and the split points only shrink)
  int fL = NG, fR = NG;
  const int QSUB = kDqWaves / a.HPW;
  const int QB = 32 * QSUB;
  const int nqb = (a.n + QB - 1) / QB;

  // block decomposition, kept scalar (the divisions run on the vector unit)
  int bid = blockIdx.x;
  const int kvh = __builtin_amdgcn_readfirstlane(bid % a.Hkv);
  bid /= a.Hkv;
  const int hg = __builtin_amdgcn_readfirstlane(bid % a.HG);
  bid /= a.HG;
  const int b = __builtin_amdgcn_readfirstlane(bid % a.B);
  bid /= a.B;
  const int qblk = __builtin_amdgcn_readfirstlane(nqb - 1 - bid);   // heaviest first
  const int n = a.n;
  const int h = __builtin_amdgcn_readfirstlane(kvh * a.r + hg * a.HPW + (wave % a.HPW));
  const int i0_wg = qblk * QB;
  const int i0w = __builtin_amdgcn_readfirstlane(i0_wg + (wave / a.HPW) * 32);
  const bool wave_valid = i0w < n;
  const int i1w = __builtin_amdgcn_readfirstlane(min(n, i0w + 32) - 1);
  const int kend = min(n, i0_wg + QB);
  const int nk = __builtin_amdgcn_readfirstlane((kend + 63) / 64);

  // Q^T and dO^T B operands, resident: lane owns query i0w + l32
  const int qi = i0w + l32;
  u32x4 qr[NCH], gr[NCH];
  {
    const u32x4 zero = {0u, 0u, 0u, 0u};
    const bf16* qp = a.q + (int64_t)b * a.qs_b + (int64_t)qi * a.qs_t + (int64_t)h * a.qs_h + hh * 8;
    const bf16* gp = a.dout + (int64_t)b * a.gs_b + (int64_t)qi * a.gs_t + (int64_t)h * a.gs_h + hh * 8;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      qr[c] = (qi < n) ? *reinterpret_cast<const u32x4*>(qp + c * 16) : zero;
      gr[c] = (qi < n) ? *reinterpret_cast<const u32x4*>(gp + c * 16) : zero;
    }
  }
  // the lane's query row: LSE in base 2 (+inf past the end: P = 0), Dsum
  float lse2 = INFINITY;
  float dsq = 0.f;
  if (qi < n) {
    const float2 rv = *reinterpret_cast<const float2*>(a.rowv + 2 * (((int64_t)b * a.Hq + h) * n + qi));
    lse2 = rv.x;
    dsq = rv.y;
  }

  const bf16* kbase = a.k + (int64_t)b * a.ks_b + (int64_t)kvh * a.ks_h;
  const bf16* vbase = a.v + (int64_t)b * a.vs_b + (int64_t)kvh * a.vs_h;
  const int krow_b = (int)(a.ks_t * 2);
  const int vrow_b = (int)(a.vs_t * 2);
  // K: read row-wise and transposed -> dual swizzle; V: row-wise only ->
  // swizzle by the row's 256-byte bank row
  int koff[LOADS], voff[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int p = (wave * LOADS + i) * 64 + lane;
    const int row = p / CPR;
    const int pc = p % CPR;
    koff[i] = row * krow_b + (pc ^ dual_swz<D>(row)) * 16;
    voff[i] = row * vrow_b + (pc ^ ((row / KRB) & (CPR - 1))) * 16;
  }
  auto load_tile = [&](int j0, int st) {
    const int rows = min(64, n - j0);          // the tile's own rows: 32-bit offsets
    const __amdgpu_buffer_rsrc_t krs =
        uniform_rsrc(kbase + (int64_t)j0 * a.ks_t, (rows - 1) * krow_b + 2 * D);
    const __amdgpu_buffer_rsrc_t vrs =
        uniform_rsrc(vbase + (int64_t)j0 * a.vs_t, (rows - 1) * vrow_b + 2 * D);
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int dst = (wave * LOADS + i) * 1024;
      dma16(krs, &smem[st][dst], koff[i]);
      dma16(vrs, &smem[st][TILE_B + dst], voff[i]);
    }
  };
  // row-wise reads of rows 32kb + l32 (the swizzles of rows 32kb + l32 do not
  // depend on kb)
  // The offset of step c is l32*RB + ((2c + hh) ^ sw) * 16; the swizzle sw
  // has at most 4 bits and the row offset starts at bit 7, so it equals
  // (l32*RB + ((hh ^ sw) & 1) * 16 + (sw >> 1) * 32) ^ (c << 5): one base
  // register per operand instead of one per step (the per-step arrays
  // spilled at d_h = 128, and every reload waited for the DMA in flight).
  int kbase_off, vbase_off;
  {
    const int swk = dual_swz<D>(l32);
    const int swv = (l32 / KRB) & (CPR - 1);
    kbase_off = l32 * RB + ((hh ^ swk) & 1) * 16 + (swk >> 1) * 32;
    vbase_off = l32 * RB + ((hh ^ swv) & 1) * 16 + (swv >> 1) * 32;
  }
  // transposing reads of K (rows 16kc + 4hh + e4 and + 8)
  const int grp = lane >> 4;
  const int e4 = (lane & 15) >> 2;
  const int q4 = lane & 3;
  int tlo[ND], thi[ND];
  {
    const int rlo = 4 * hh + e4, rhi = rlo + 8;
#pragma unroll
    for (int db = 0; db < ND; ++db) {
      const int chunk = 4 * db + 2 * (grp & 1) + (q4 >> 1);
      tlo[db] = rlo * RB + (chunk ^ dual_swz<D>(rlo)) * 16 + (q4 & 1) * 8;
      thi[db] = rhi * RB + (chunk ^ dual_swz<D>(rhi)) * 16 + (q4 & 1) * 8;
    }
  }

  const f32x16 zero16 = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  f32x16 dqt[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db) dqt[db] = zero16;
  const float sl2 = a.scale_log2;

  load_tile(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  for (int it = 0; it < nk; ++it) {
    const int j0 = it * 64;
    const int st = it & 1;
    if (it + 1 < nk) load_tile(j0 + 64, st ^ 1);
    const unsigned char* sk = &smem[st][0];
    const unsigned char* sv = &smem[st][TILE_B];
    if (wave_valid && j0 <= i1w) {
      const int j1 = min(n - 1, j0 + 63);
      int sL, sR;
      if constexpr (FINE) {
        const int lD = max(0, i0w - j1), rD = i1w - j0;
        while (fL > 0 && cut_at(fL - 1) >= lD) --fL;
        while (fR > 0 && cut_at(fR - 1) >= rD) --fR;
        sL = fL;
        sR = fR;
      } else {
        split_points<NG>(a.cut, max(0, i0w - j1), i1w - j0, sL, sR);
      }
      // the bases are re-declared live here each tile, so that the compiler
      // forms the per-step offsets at their use instead of hoisting eight of
      // each out of the loop
      asm volatile("" : "+v"(kbase_off), "+v"(vbase_off));
      auto kop = [&](int kb, int c) {
        return *reinterpret_cast<const u32x4*>(sk + kb * 32 * RB + (kbase_off ^ (c << 5)));
      };
      auto vop = [&](int kb, int c) {
        return *reinterpret_cast<const u32x4*>(sv + kb * 32 * RB + (vbase_off ^ (c << 5)));
      };
      const int base = qi - j0;                    // distance = base - (32kb + out_row(r))

      u32x4 dsp[4];                                // dS^T as B operands, 16 keys each
      f32x16 dsv[2];                               // dS^T values (for partial-group masks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        // ---- S^T = K Q^T: full groups as one chain, then partials ----
        f32x16 s = zero16;
        if constexpr (FINE) {
          // as in the dK/dV kernel: a chain over the all-full steps, then
          // the mixed steps with operand words zeroed per group
          const int c_end = (sR * G + 15) / 16;
          const int c_lo = (sL * G) / 16;
          if (c_end < NCH) {
            s = mfma32(kop(kb, NCH - 1), qr[NCH - 1], zero16);
#pragma unroll
            for (int cc = NCH - 2; cc >= 0; --cc) {
              if (cc < c_end) break;
              s = mfma32(kop(kb, cc), qr[cc], s);
            }
          }
#pragma unroll
          for (int c = 0; c < NCH; ++c) {
            if (c < c_lo || c >= c_end) continue;
            const u32x4 ka = kop(kb, c);
            auto grp = [&](int w) { return (16 * c + 8 * hh + 2 * w) / G; };
            if ((16 * c + 15) / G >= sR) s = mfma32(ka, keep_words(qr[c], [&](int w) { return grp(w) >= sR; }), s);
#pragma unroll 1
            for (int g = max((16 * c) / G, sL); g < min((16 * c + 15) / G + 1, sR); ++g) {
              const int cg = cut_at(g);
              const f32x16 t = mfma32(ka, keep_words(qr[c], [&](int w) { return grp(w) == g; }), zero16);
#pragma unroll
              for (int r = 0; r < 16; ++r) s[r] += (base - 32 * kb - out_row(r, hh) <= cg) ? t[r] : 0.f;
            }
          }
        } else {
        if (sR < NG) {
          s = mfma32(kop(kb, NCH - 1), qr[NCH - 1], zero16);
#pragma unroll
          for (int cc = NCH - 2; cc >= 0; --cc) {
            if (cc < sR * GC) break;
            s = mfma32(kop(kb, cc), qr[cc], s);
          }
        }
        if (sL < sR) {
#pragma unroll
          for (int g = NG - 1; g >= 0; --g) {
            if (g >= sR || g < sL) continue;
            f32x16 t = zero16;
#pragma unroll
            for (int c = 0; c < GC; ++c) t = mfma32(kop(kb, g * GC + c), qr[g * GC + c], t);
#pragma unroll
            for (int r = 0; r < 16; ++r) s[r] += (base - 32 * kb - out_row(r, hh) <= a.cut[g]) ? t[r] : 0.f;
          }
        }
        }
        // ---- dP^T = V dO^T ----
        f32x16 dp = mfma32(vop(kb, 0), gr[0], zero16);
#pragma unroll
        for (int c = 1; c < NCH; ++c) dp = mfma32(vop(kb, c), gr[c], dp);
        // ---- P^T, dS^T; keys after the query are masked, on the key
        //      blocks that reach past the wave's first query ----
        f32x16 pr;
#pragma unroll
        for (int r = 0; r < 16; ++r) pr[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], sl2, -lse2));
        if (j0 + 32 * kb + 31 > i0w) {
#pragma unroll
          for (int r = 0; r < 16; ++r) pr[r] = (base - 32 * kb - out_row(r, hh) >= 0) ? pr[r] : 0.f;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) dsv[kb][r] = pr[r] * (dp[r] - dsq);
        u32x4 pk[2];
        pack_block(dsv[kb], pk);
        dsp[2 * kb] = pk[0];
        dsp[2 * kb + 1] = pk[1];
      }

      // ---- dQ^T += K^T dS^T, masked per group ----
      if constexpr (FINE) {
        // per 32-dim block: its full groups with unmasked dS^T and the A rows
        // (dims) of other groups zeroed, then a run-time loop over its
        // partial groups, each with dS^T masked by the group's cutoff and
        // the A rows of the group only
#pragma unroll
        for (int db = 0; db < ND; ++db) {
          const int ga = (32 * db) / G, gb = (32 * db + 31) / G;
          if (gb < sL) continue;                     // every group of the block skipped
          const int gl = (32 * db + l32) / G;        // group of this lane's A row
          u32x4 ka[4];
#pragma unroll
          for (int kc = 0; kc < 4; ++kc) {
            const u32x2 lo = read_tr16(sk + kc * 16 * RB + tlo[db]);
            const u32x2 hi = read_tr16(sk + kc * 16 * RB + thi[db]);
            ka[kc] = u32x4{lo[0], lo[1], hi[0], hi[1]};
          }
          if (gb >= sR) {
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) dqt[db] = mfma32(gl >= sR ? ka[kc] : zero4, dsp[kc], dqt[db]);
          }
#pragma unroll 1
          for (int g = max(ga, sL); g < min(gb + 1, sR); ++g) {
            const int cg = cut_at(g);
            u32x4 bop[4];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
              f32x16 dm;
#pragma unroll
              for (int r = 0; r < 16; ++r) dm[r] = (base - 32 * kb - out_row(r, hh) <= cg) ? dsv[kb][r] : 0.f;
              u32x4 pk[2];
              pack_block(dm, pk);
              bop[2 * kb] = pk[0];
              bop[2 * kb + 1] = pk[1];
            }
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) dqt[db] = mfma32(gl == g ? ka[kc] : zero4, bop[kc], dqt[db]);
          }
        }
      } else {
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        const int ga = (32 * db) / G, gb = (32 * db + 31) / G;
        if (ga >= sR) {
#pragma unroll
          for (int kc = 0; kc < 4; ++kc) {
            const u32x2 lo = read_tr16(sk + kc * 16 * RB + tlo[db]);
            const u32x2 hi = read_tr16(sk + kc * 16 * RB + thi[db]);
            dqt[db] = mfma32(u32x4{lo[0], lo[1], hi[0], hi[1]}, dsp[kc], dqt[db]);
          }
        } else {
#pragma unroll
          for (int g = ga; g <= gb; ++g) {
            if (g < sL) continue;
            u32x4 bop[4];
            if (g >= sR) {
#pragma unroll
              for (int kc = 0; kc < 4; ++kc) bop[kc] = dsp[kc];
            } else {
              const int cg = a.cut[g];
#pragma unroll
              for (int kb = 0; kb < 2; ++kb) {
                f32x16 dm;
#pragma unroll
                for (int r = 0; r < 16; ++r)
                  dm[r] = (base - 32 * kb - out_row(r, hh) <= cg) ? dsv[kb][r] : 0.f;
                u32x4 pk[2];
                pack_block(dm, pk);
                bop[2 * kb] = pk[0];
                bop[2 * kb + 1] = pk[1];
              }
            }
            const bool mine = ((32 * db + l32) / G) == g;
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) {
              const u32x2 lo = read_tr16(sk + kc * 16 * RB + tlo[db]);
              const u32x2 hi = read_tr16(sk + kc * 16 * RB + thi[db]);
              const u32x4 aop = mine ? u32x4{lo[0], lo[1], hi[0], hi[1]} : zero4;
              dqt[db] = mfma32(aop, bop[kc], dqt[db]);
            }
          }
        }
      }
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }

  // ---- dQ = scale * dQ^T: lane's query, rows = dims ----
  if (wave_valid && qi < n) {
    bf16* qp = a.dq + (int64_t)b * a.dqs_b + (int64_t)qi * a.dqs_t + (int64_t)h * a.dqs_h + hh * 4;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        u32x2 w;
        w[0] = pack_bf16x2(dqt[db][4 * r4] * a.scale, dqt[db][4 * r4 + 1] * a.scale);
        w[1] = pack_bf16x2(dqt[db][4 * r4 + 2] * a.scale, dqt[db][4 * r4 + 3] * a.scale);
        *reinterpret_cast<u32x2*>(qp + db * 32 + r4 * 8) = w;
      }
  }
}

template <int D, int G>
hipError_t launch_bwd(const BackwardArgs& a, hipStream_t s) {
  const long long rows = (long long)a.B * a.n * a.Hq;
  hipLaunchKernelGGL((bwd_dsum_kernel<D>), dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long kblocks = (long long)a.Hkv * a.B * ((a.n + 127) / 128);
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, G>), dim3((unsigned)kblocks), dim3(kKvThreads), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int QB = 32 * (kDqWaves / a.HPW);
  const long long qblocks = (long long)a.Hkv * a.HG * a.B * ((a.n + QB - 1) / QB);
  hipLaunchKernelGGL((bwd_dq_kernel<D, G>), dim3((unsigned)qblocks), dim3(kDqThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_backward(const BackwardArgs& a, int d_h, int G, hipStream_t s) {
  if (a.B < 1 || a.n < 1) return hipSuccess;
  if (d_h == 128 && G == 16) return launch_bwd<128, 16>(a, s);
  if (d_h == 128 && G == 32) return launch_bwd<128, 32>(a, s);
  if (d_h == 64 && G == 16) return launch_bwd<64, 16>(a, s);
  if (d_h == 64 && G == 32) return launch_bwd<64, 32>(a, s);
  if (d_h == 128 && G == 8) return launch_bwd<128, 8>(a, s);
  if (d_h == 128 && G == 4) return launch_bwd<128, 4>(a, s);
  if (d_h == 128 && G == 2) return launch_bwd<128, 2>(a, s);
  if (d_h == 64 && G == 8) return launch_bwd<64, 8>(a, s);
  if (d_h == 64 && G == 4) return launch_bwd<64, 4>(a, s);
  if (d_h == 64 && G == 2) return launch_bwd<64, 2>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace wp
