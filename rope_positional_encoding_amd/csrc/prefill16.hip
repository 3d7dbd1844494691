// WavePrune causal prefill attention for gfx950 on v_mfma_f32_16x16x32_bf16:
// the 32-dim group variant (G = 32, d_h = 128) and its dense baseline.
//
// Same method, tiling and staging as prefill.hip (grouped rule of the
// WavePrune reading notes on cc.laoqi.cc, section 2.3, Eq. (8); tile classes
// from the section 2.3 table), with the 16x16x32 MFMA instead of 32x32x16:
//  * One MFMA contracts 32 head dims -- exactly one G = 32 group -- so the
//    full groups [splitR, 4) are a chain of whole steps and a partial group
//    is one masked step.
//  * A wave still owns 32 queries x 64 keys, now as 2 x 4 output blocks of
//    16 x 16.  S^T = K Q^T: the K operand (16 keys x 32 dims, one 16-byte
//    LDS read per lane) feeds the MFMAs of both 16-query blocks; a lane holds
//    two query columns (its own in each block) and, per block, 4 keys of each
//    16-key block.  Row max / row sum reduce over the 4 lane quarters with
//    v_permlane16_swap and v_permlane32_swap.
//  * O^T += V^T P^T with 8 blocks of 16 dims: the P^T operand of a 32-key
//    chunk is the lane's own probabilities (keys 4q..4q+3 of both 16-key
//    blocks of the chunk) and the V^T operand is two transposing LDS reads
//    (ds_read_b64_tr_b16) of the same keys, so no data moves between lanes.
//  * K rows are XOR-swizzled in LDS by (row & 15) (16 rows read at one
//    logical chunk hit 16 distinct chunks), V rows by 2 (row & 7), which
//    keeps each 32-lane half of a transposing read on distinct banks.
// Every FLOP and byte per tile equals the 32x32x16 kernel's; the 16x16x32
// MFMA takes 16 cycles for half the work of a 32-cycle 32x32x16 one.
#include "wp_device.h"
#include "wp_internal.h"

namespace wp {

namespace {

constexpr int kThreads16 = 512;
constexpr int kWaves16 = 8;
constexpr int kTile16 = 64;      // keys per tile (four 16-key blocks, one class per group)

__device__ inline f32x4 mfma16x32(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

// max / sum over the four lane quarters (lanes l, l^16, l^32, l^48), which
// hold the same query column
__device__ inline float quad_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return halves_max(fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}
__device__ inline float quad_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return halves_sum(__uint_as_float(r[0]) + __uint_as_float(r[1]));
}

// The four K operands (key blocks 0-3) of one S^T step, complete on return;
// one asm block with its own wait, issued after the previous step's MFMAs.
__device__ inline void k_reads4(u32x4& a, u32x4& b, u32x4& c, u32x4& d, unsigned addr) {
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %4 offset:4096\n\t"
      "ds_read_b128 %2, %4 offset:8192\n\t"
      "ds_read_b128 %3, %4 offset:12288\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(a), "=&v"(b), "=&v"(c), "=&v"(d)
      : "v"(addr)
      : "memory");
}

template <bool COUNT>
__global__ __launch_bounds__(kThreads16) void prefill16_kernel(PrefillArgs a) {
  constexpr int D = 128;
  constexpr int NS = D / 32;            // 32-dim MFMA steps = groups
  constexpr int NG = 4;
  constexpr int NDB = D / 16;           // 16-dim output blocks
  constexpr int RB = D * 2;             // bytes per K/V row in LDS
  constexpr int CPR = D / 8;            // 16-byte chunks per row
  constexpr int TILE_B = kTile16 * RB;
  constexpr int LOADS = TILE_B / (kWaves16 * 64 * 16);
  static_assert(LOADS == 2, "tile shape");

  __shared__ __attribute__((aligned(1024))) unsigned char smem[2][2 * TILE_B];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15;
  const int g4 = lane >> 4;

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
  const int i0w = __builtin_amdgcn_readfirstlane(i0_wg + (wave / a.HPW) * 32);
  const bool wave_valid = i0w < n;
  const int i1w = __builtin_amdgcn_readfirstlane(min(n, i0w + 32) - 1);
  const int kend = min(n, i0_wg + a.QB);
  const int nk = __builtin_amdgcn_readfirstlane((kend + kTile16 - 1) / kTile16);

  const bf16* kbase = a.k + (int64_t)b * a.ks_b + (int64_t)kvh * a.ks_h;
  const bf16* vbase = a.v + (int64_t)b * a.vs_b + (int64_t)kvh * a.vs_h;
  const int krow_b = (int)(a.ks_t * 2);
  const int vrow_b = (int)(a.vs_t * 2);

  // Q^T operands: block qb, step c -> query i0w + 16 qb + l16, dims
  // [32c + 8 g4, 32c + 8 g4 + 8)
  u32x4 qr[2][NS];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int i = i0w + 16 * qb + l16;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    const bf16* qp = a.q + (int64_t)b * a.qs_b + (int64_t)i * a.qs_t + (int64_t)h * a.qs_h + g4 * 8;
#pragma unroll
    for (int c = 0; c < NS; ++c) qr[qb][c] = (i < n) ? *reinterpret_cast<const u32x4*>(qp + c * 32) : zero;
  }

  // ---- DMA: load i of this wave fills LDS chunks p = (wave*LOADS + i)*64 +
  //      lane of the tile, row p / CPR; physical chunk pc holds logical chunk
  //      pc ^ (row & 15) (K) or pc ^ 2 (row & 7) (V) ----
  int koff[LOADS], voff[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int p = (wave * LOADS + i) * 64 + lane;
    const int row = p / CPR;
    const int pc = p % CPR;
    koff[i] = row * krow_b + (pc ^ (row & 15)) * 16;
    voff[i] = row * vrow_b + (pc ^ (2 * (row & 7))) * 16;
  }
  auto load_tile = [&](int j0, int stage) {
    const int rows = min(kTile16, n - j0);    // the tile's own rows: 32-bit offsets
    const __amdgpu_buffer_rsrc_t kr = uniform_rsrc(kbase + (int64_t)j0 * a.ks_t, (rows - 1) * krow_b + 2 * D);
    const __amdgpu_buffer_rsrc_t vr = uniform_rsrc(vbase + (int64_t)j0 * a.vs_t, (rows - 1) * vrow_b + 2 * D);
    unsigned char* kdst = &smem[stage][0];
    unsigned char* vdst = &smem[stage][TILE_B];
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int dst = (wave * LOADS + i) * 1024;
      dma16(kr, kdst + dst, koff[i]);
      dma16(vr, vdst + dst, voff[i]);
    }
  };

  // ---- LDS read offsets.  K operand of (key block kb, step c): row
  //      16 kb + l16, logical chunk 4c + g4.  V^T operand of (output block
  //      db, 32-key chunk kc): two transposing reads, keys
  //      32 kc + 4 g4 + e and 32 kc + 16 + 4 g4 + e at dims 16 db + 4q .. ----
  int kread[NS];
#pragma unroll
  for (int c = 0; c < NS; ++c) kread[c] = l16 * RB + (((4 * c + g4) ^ l16) * 16);
  const int e4 = l16 >> 2;
  const int q4 = l16 & 3;
  int vread[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int row = 4 * g4 + e4;
    vread[db] = row * RB + (((2 * db + (q4 >> 1)) ^ (2 * (row & 7))) * 16) + (q4 & 1) * 8;
  }

  float m_i[2] = {-INFINITY, -INFINITY};   // running max per query block (log2), stale by < 8
  float l_i[2] = {0.f, 0.f};               // running sum (this lane's quarter of the keys)
  const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
  f32x4 o[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db][0] = o[db][1] = z4;

  unsigned int cnt[NG][3];
  unsigned int cnt_vis = 0;
  if (COUNT) {
#pragma unroll
    for (int g = 0; g < NG; ++g) cnt[g][0] = cnt[g][1] = cnt[g][2] = 0;
  }
  const float sl2 = a.scale_log2;

  load_tile(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  for (int it = 0; it < nk; ++it) {
    const int j0 = it * kTile16;
    const int stage = it & 1;
    if (it + 1 < nk) load_tile(j0 + kTile16, stage ^ 1);
    const unsigned char* sk = &smem[stage][0];
    const unsigned char* sv = &smem[stage][TILE_B];
    if (wave_valid && j0 <= i1w) {
      // ---- classify the (32 queries x 64 keys) tile ----
      const int j1 = min(n - 1, j0 + kTile16 - 1);
      const int lD = max(0, i0w - j1);
      const int rD = i1w - j0;
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

      // ---- S^T = K Q^T: full groups [sR, 4) as one descending chain; the K
      //      operands of step c-1 are read right after step c's MFMAs ----
      f32x4 s[4][2];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) s[kb][0] = s[kb][1] = z4;
      if (sR < NS) {
        const unsigned skb = lds_addr(sk);
        u32x4 k0, k1, k2, k3;
        k_reads4(k0, k1, k2, k3, skb + kread[NS - 1]);
#pragma unroll
        for (int c = NS - 1; c >= 0; --c) {
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            s[0][qb] = mfma16x32(k0, qr[qb][c], s[0][qb]);
            s[1][qb] = mfma16x32(k1, qr[qb][c], s[1][qb]);
            s[2][qb] = mfma16x32(k2, qr[qb][c], s[2][qb]);
            s[3][qb] = mfma16x32(k3, qr[qb][c], s[3][qb]);
          }
          if (c == sR) break;
          __builtin_amdgcn_sched_barrier(0);
          k_reads4(k0, k1, k2, k3, skb + kread[c - 1]);
        }
      }
      // dist of (block kb, qb, register r) = base + 16 qb - 16 kb - r
      const int base = (i0w + l16) - (j0 + 4 * g4);
      if (sL < sR) {
        // ---- partial groups: one masked step each ----
#pragma unroll
        for (int g = NG - 1; g >= 0; --g) {
          if (g >= sR || g < sL) continue;
          const int cg = a.cut[g];
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            const u32x4 kk = *reinterpret_cast<const u32x4*>(sk + kb * 16 * RB + kread[g]);
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
              const f32x4 t = mfma16x32(kk, qr[qb][g], z4);
#pragma unroll
              for (int r = 0; r < 4; ++r) s[kb][qb][r] += (base + 16 * qb - 16 * kb - r <= cg) ? t[r] : 0.f;
            }
          }
        }
      }
      // ---- causal mask on tiles that reach past the wave's first query ----
      if (j0 + kTile16 - 1 > i0w) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (base + 16 * qb - 16 * kb - r < 0) s[kb][qb][r] = -INFINITY;
      }

      // ---- online softmax per query block, log2 domain, lazy rescale ----
      float mc[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        float m4[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
          m4[kb] = fmaxf(fmaxf(s[kb][qb][0], s[kb][qb][1]), fmaxf(s[kb][qb][2], s[kb][qb][3]));
        mc[qb] = quad_max(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]))) * sl2;
      }
      if (__any(mc[0] > m_i[0] + 8.f || mc[1] > m_i[1] + 8.f)) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const float m_new = fmaxf(m_i[qb], mc[qb]);
          const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
          const float alpha = __builtin_amdgcn_exp2f(m_i[qb] - m_use);
          l_i[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < NDB; ++db) o[db][qb] *= alpha;
          m_i[qb] = m_use;
        }
      }
      // P^T operand of (qb, 32-key chunk kc): keys 32kc + 4g4 + r of block
      // 2kc, then of block 2kc + 1
      u32x4 p[2][2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][qb][0], sl2, -m_i[qb]));
          const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][qb][1], sl2, -m_i[qb]));
          const float e2 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][qb][2], sl2, -m_i[qb]));
          const float e3 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][qb][3], sl2, -m_i[qb]));
          l_i[qb] += (e0 + e1) + (e2 + e3);
          p[qb][kb >> 1][2 * (kb & 1)] = pack_bf16x2(e0, e1);
          p[qb][kb >> 1][2 * (kb & 1) + 1] = pack_bf16x2(e2, e3);
        }

      // ---- O^T += V^T P^T: each V^T operand feeds both query blocks ----
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const unsigned char* va = sv + kc * 32 * RB + vread[db];
          const u32x2 lo2 = read_tr16(va);
          const u32x2 hi2 = read_tr16(va + 16 * RB);
          const u32x4 vop = {lo2[0], lo2[1], hi2[0], hi2[1]};
          o[db][0] = mfma16x32(vop, p[0][kc], o[db][0]);
          o[db][1] = mfma16x32(vop, p[1][kc], o[db][1]);
        }
    }
    // tile it+1 must be in LDS, and every wave done with stage it&1, before
    // the next iteration
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }

  if (wave_valid) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float l_tot = quad_sum(l_i[qb]);
      const int i = i0w + 16 * qb + l16;
      if (i < n) {
        const float inv = 1.f / l_tot;
        bf16* op = a.o + (int64_t)b * a.os_b + (int64_t)i * a.os_t + (int64_t)h * a.os_h + 4 * g4;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          u32x2 w;
          w[0] = pack_bf16x2(o[db][qb][0] * inv, o[db][qb][1] * inv);
          w[1] = pack_bf16x2(o[db][qb][2] * inv, o[db][qb][3] * inv);
          *reinterpret_cast<u32x2*>(op + 16 * db) = w;
        }
        if (a.lse && g4 == 0)
          a.lse[((int64_t)b * a.Hq + h) * n + i] = (m_i[qb] + __log2f(l_tot)) * 0.69314718055994531f;
      }
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

}  // namespace

hipError_t launch_prefill16(const PrefillArgs& a0, bool count, hipStream_t s) {
  // each wave takes 32 queries of one head: HPW heads x QSUB query blocks
  PrefillArgs a = a0;
  a.QSUB = kWaves16 / a.HPW;
  a.QB = 32 * a.QSUB;
  a.nqb = (a.n + a.QB - 1) / a.QB;
  const long long blocks = (long long)a.B * a.Hkv * a.HG * a.nqb;
  if (blocks <= 0) return hipSuccess;
  if (count)
    hipLaunchKernelGGL(prefill16_kernel<true>, dim3((unsigned)blocks), dim3(kThreads16), 0, s, a);
  else
    hipLaunchKernelGGL(prefill16_kernel<false>, dim3((unsigned)blocks), dim3(kThreads16), 0, s, a);
  return hipGetLastError();
}

}  // namespace wp
