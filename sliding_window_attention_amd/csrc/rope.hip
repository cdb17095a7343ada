// rope.hip — rotary position embedding (rotate-half form) of a [B, T, H, D]
// tensor, used to rotate the keys once before the banded prefill (the queries
// are rotated in registers inside the prefill kernel).
//
// The pair (x_i, x_{i+D/2}) of a token at position p turns by the angle
// p * base^(-2i/D) ([G3] "How it works": base 1e4 on local layers; [KB] §2
// "Interleaved local/global schemes": 1e4 local / 1e6 global).  The angle is
// formed in float64 revolutions and reduced to [0, 1) before the float32
// sine and cosine.
//
// Tags: [KB] knowledge-base page "Sliding Window Attention" (lizeman.github.io);
// [G3] "Sliding Window Attention — Gemma 3" study note (ai-engineer-exhaustive.pages.dev).

#include <cmath>

#include "swa_internal.h"

namespace swa {
namespace {

// Each thread rotates 8 consecutive pairs (i0 .. i0+7, i0 a multiple of 8) of
// one row per step: one 16-byte (bf16) or two 16-byte (fp32) accesses per
// half-row, threads of a row side by side, so a wave reads whole rows.  The
// pair rates rev0 * step^i are formed once per thread.  y may alias x (each
// thread reads its elements before writing them).
template <bool F32>
__global__ __launch_bounds__(256) void rope_kernel(const void *x, void *y, const int *pos, int T,
                                                  int H, int D, long long rows, double rev0,
                                                  double step) {
  const int half = D / 2;
  const int tpr = half / 8;  // threads per row
  const int i0 = (threadIdx.x % tpr) * 8;
  const int rpb = 256 / tpr;  // rows per block step
  double rv[8];
  rv[0] = rev0 * rope_pow(step, i0);
#pragma unroll
  for (int e = 1; e < 8; ++e) rv[e] = rv[e - 1] * step;
  for (long long row = (long long)blockIdx.x * rpb + threadIdx.x / tpr; row < rows;
       row += (long long)gridDim.x * rpb) {
    const long long bt = row / H;  // (b, t) of this row
    const double p = pos ? (double)pos[bt] : (double)(int)(bt % T);
    const long long o0 = row * D + i0, o1 = o0 + half;
    float a[8], b[8];
    if constexpr (F32) {
      const float4 *xa = reinterpret_cast<const float4 *>(static_cast<const float *>(x) + o0);
      const float4 *xb = reinterpret_cast<const float4 *>(static_cast<const float *>(x) + o1);
      const float4 a0 = xa[0], a1 = xa[1], b0 = xb[0], b1 = xb[1];
      a[0] = a0.x; a[1] = a0.y; a[2] = a0.z; a[3] = a0.w;
      a[4] = a1.x; a[5] = a1.y; a[6] = a1.z; a[7] = a1.w;
      b[0] = b0.x; b[1] = b0.y; b[2] = b0.z; b[3] = b0.w;
      b[4] = b1.x; b[5] = b1.y; b[6] = b1.z; b[7] = b1.w;
    } else {
      const uint4 ua = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(x) + o0);
      const uint4 ub = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(x) + o1);
      const uint32_t wa[4] = {ua.x, ua.y, ua.z, ua.w}, wb[4] = {ub.x, ub.y, ub.z, ub.w};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        a[2 * w] = __uint_as_float(wa[w] << 16);
        a[2 * w + 1] = __uint_as_float(wa[w] & 0xffff0000u);
        b[2 * w] = __uint_as_float(wb[w] << 16);
        b[2 * w + 1] = __uint_as_float(wb[w] & 0xffff0000u);
      }
    }
    float ra[8], rb[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double xr = p * rv[e];
      float sn, cs;
      sincosf((float)((xr - floor(xr)) * 6.283185307179586), &sn, &cs);
      ra[e] = a[e] * cs - b[e] * sn;
      rb[e] = b[e] * cs + a[e] * sn;
    }
    if constexpr (F32) {
      float4 *ya = reinterpret_cast<float4 *>(static_cast<float *>(y) + o0);
      float4 *yb = reinterpret_cast<float4 *>(static_cast<float *>(y) + o1);
      ya[0] = make_float4(ra[0], ra[1], ra[2], ra[3]);
      ya[1] = make_float4(ra[4], ra[5], ra[6], ra[7]);
      yb[0] = make_float4(rb[0], rb[1], rb[2], rb[3]);
      yb[1] = make_float4(rb[4], rb[5], rb[6], rb[7]);
    } else {
      uint32_t wa[4], wb[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const __bf16 a0 = (__bf16)ra[2 * w], a1 = (__bf16)ra[2 * w + 1];
        const __bf16 b0 = (__bf16)rb[2 * w], b1 = (__bf16)rb[2 * w + 1];
        wa[w] = (uint32_t)__builtin_bit_cast(uint16_t, a0) |
                ((uint32_t)__builtin_bit_cast(uint16_t, a1) << 16);
        wb[w] = (uint32_t)__builtin_bit_cast(uint16_t, b0) |
                ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
      }
      *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(y) + o0) = make_uint4(wa[0], wa[1], wa[2], wa[3]);
      *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(y) + o1) = make_uint4(wb[0], wb[1], wb[2], wb[3]);
    }
  }
}

}  // namespace

hipError_t launch_rope(bool f32, const void *x, void *y, const int *pos, int B, int T, int H, int D,
                       double rev0, double step, hipStream_t st) {
  const long long rows = (long long)B * T * H;
  const int rpb = 256 / (D / 16);  // rows per block step: 8 pairs per thread
  long long blocks = (rows + rpb - 1) / rpb;
  if (blocks > 8192) blocks = 8192;
  if (blocks <= 0) return hipSuccess;
  if (f32)
    hipLaunchKernelGGL(rope_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, st, x, y, pos, T, H,
                       D, rows, rev0, step);
  else
    hipLaunchKernelGGL(rope_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, st, x, y, pos, T,
                       H, D, rows, rev0, step);
  return hipGetLastError();
}

}  // namespace swa
