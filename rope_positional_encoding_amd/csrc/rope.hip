// RoPE application for gfx950: rotate every interleaved channel pair
// (2c, 2c+1) of every head by p * f_c, f_c = theta^(-2c/d_h) / pos_scale.
// The rotation is the standard 2x2 matrix [[cos, -sin], [sin, cos]]
// (WavePrune reading notes on cc.laoqi.cc, section 1.1; the rotation matrix in
// the kongchang.com article's RoPE paragraph).
//
// HBM-bound: one read and one write per element.  The angles depend on
// (token, channel) only, so a workgroup first fills an LDS table of
// (cos, sin) for its token rows -- the angle is formed and reduced modulo
// 2*pi in float64, so positions up to 2^31 keep full float32 accuracy -- and
// then streams every head of those rows through it in 16-byte chunks.
#include "wp_internal.h"

namespace wp {

namespace {

constexpr int kRopeThreads = 256;
constexpr int kRopeMaxRows = 32;

__device__ inline float bf16_lo(unsigned int w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(unsigned int w) { return __uint_as_float(w & 0xffff0000u); }

__device__ inline unsigned int pack_bf16x2(float lo, float hi) {
  const __bf16 a = static_cast<__bf16>(lo);
  const __bf16 b = static_cast<__bf16>(hi);
  return (unsigned int)__builtin_bit_cast(unsigned short, a) |
         ((unsigned int)__builtin_bit_cast(unsigned short, b) << 16);
}

__global__ __launch_bounds__(kRopeThreads) void rope_kernel(RopeArgs a) {
  __shared__ float2 cs[kRopeMaxRows * kMaxChannels];
  const int C = a.d_h >> 1;
  const int CH = a.d_h >> 3;                    // 8-dim chunks per head
  const int64_t nrows = (int64_t)a.B * a.n;
  const int64_t row0 = (int64_t)blockIdx.x * a.rows_per_block;

  // (cos, sin) for every (row, channel) of this block
  for (int idx = threadIdx.x; idx < a.rows_per_block * C; idx += kRopeThreads) {
    const int rr = idx / C;
    const int c = idx - rr * C;
    const int64_t row = row0 + rr;
    if (row >= nrows) continue;
    const int b = (int)(row / a.n);
    const int t = (int)(row - (int64_t)b * a.n);
    const double p = (double)t + (a.pos_start ? (double)a.pos_start[b] : 0.0);
    const double ang = p * a.inv_freq[c];
    const double turns = rint(ang * 0.15915494309189535);   // 1 / (2 pi)
    const double red = fma(-turns, 6.283185307179586, ang);
    float s, co;
    sincosf((float)red, &s, &co);
    cs[rr * kMaxChannels + c] = make_float2(co, s);
  }
  __syncthreads();

  const int items = a.rows_per_block * a.H * CH;
  for (int idx = threadIdx.x; idx < items; idx += kRopeThreads) {
    const int ch = idx % CH;
    const int rest = idx / CH;
    const int h = rest % a.H;
    const int rr = rest / a.H;
    const int64_t row = row0 + rr;
    if (row >= nrows) continue;
    const int64_t b = row / a.n;
    const int64_t t = row - b * a.n;
    float x[8];
    if (a.x_f32) {
      const float* src = reinterpret_cast<const float*>(a.x) + b * a.xs_b + t * a.xs_t +
                         h * a.xs_h + ch * 8;
      const f32x4 u = *reinterpret_cast<const f32x4*>(src);
      const f32x4 w = *reinterpret_cast<const f32x4*>(src + 4);
      x[0] = u[0]; x[1] = u[1]; x[2] = u[2]; x[3] = u[3];
      x[4] = w[0]; x[5] = w[1]; x[6] = w[2]; x[7] = w[3];
    } else {
      const bf16* src = reinterpret_cast<const bf16*>(a.x) + b * a.xs_b + t * a.xs_t +
                        h * a.xs_h + ch * 8;
      const u32x4 u = *reinterpret_cast<const u32x4*>(src);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[2 * e] = bf16_lo(u[e]);
        x[2 * e + 1] = bf16_hi(u[e]);
      }
    }
    u32x4 out;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float2 r = cs[rr * kMaxChannels + ch * 4 + e];
      const float x0 = x[2 * e], x1 = x[2 * e + 1];
      out[e] = pack_bf16x2(x0 * r.x - x1 * r.y, x0 * r.y + x1 * r.x);
    }
    bf16* dst = reinterpret_cast<bf16*>(a.y) + b * a.ys_b + t * a.ys_t + h * a.ys_h + ch * 8;
    *reinterpret_cast<u32x4*>(dst) = out;
  }
}

}  // namespace

hipError_t launch_rope(const RopeArgs& a_in, hipStream_t s) {
  RopeArgs a = a_in;
  const int per_row = a.H * (a.d_h / 8);
  int rows = 1024 / (per_row > 0 ? per_row : 1);
  if (rows < 1) rows = 1;
  if (rows > kRopeMaxRows) rows = kRopeMaxRows;
  a.rows_per_block = rows;
  const int64_t nrows = (int64_t)a.B * a.n;
  const int64_t blocks = (nrows + rows - 1) / rows;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(rope_kernel, dim3((unsigned)blocks), dim3(kRopeThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace wp
