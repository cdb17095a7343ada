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

// Block: D/2 pair columns x (256 / (D/2)) rows per step; the pair's revolution
// rate rev0 * step^i is computed once per thread.  y may alias x (each thread
// reads both elements of its pair before writing them).
template <bool F32>
__global__ __launch_bounds__(256) void rope_kernel(const void *x, void *y, const int *pos, int T,
                                                  int H, int D, long long rows, double rev0,
                                                  double step) {
  const int half = D / 2;
  const int i = threadIdx.x % half;
  const int rpb = 256 / half;  // rows per block step
  const double rev_i = rev0 * rope_pow(step, i);
  for (long long row = (long long)blockIdx.x * rpb + threadIdx.x / half; row < rows;
       row += (long long)gridDim.x * rpb) {
    const long long bt = row / H;  // (b, t) of this row
    const int t = (int)(bt % T);
    const double p = pos ? (double)pos[bt] : (double)t;
    const double xr = p * rev_i;
    const float ang = (float)((xr - floor(xr)) * 6.283185307179586);
    float sn, cs;
    sincosf(ang, &sn, &cs);
    const long long o0 = row * D + i, o1 = o0 + half;
    if constexpr (F32) {
      const float a = static_cast<const float *>(x)[o0], b = static_cast<const float *>(x)[o1];
      static_cast<float *>(y)[o0] = a * cs - b * sn;
      static_cast<float *>(y)[o1] = b * cs + a * sn;
    } else {
      const uint16_t ua = static_cast<const uint16_t *>(x)[o0];
      const uint16_t ub = static_cast<const uint16_t *>(x)[o1];
      const float a = __uint_as_float((uint32_t)ua << 16), b = __uint_as_float((uint32_t)ub << 16);
      const __bf16 ra = (__bf16)(a * cs - b * sn), rb = (__bf16)(b * cs + a * sn);
      static_cast<uint16_t *>(y)[o0] = __builtin_bit_cast(uint16_t, ra);
      static_cast<uint16_t *>(y)[o1] = __builtin_bit_cast(uint16_t, rb);
    }
  }
}

}  // namespace

hipError_t launch_rope(bool f32, const void *x, void *y, const int *pos, int B, int T, int H, int D,
                       double rev0, double step, hipStream_t st) {
  const long long rows = (long long)B * T * H;
  const int rpb = 256 / (D / 2);
  long long blocks = (rows + rpb - 1) / rpb;
  if (blocks > 65536) blocks = 65536;
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
