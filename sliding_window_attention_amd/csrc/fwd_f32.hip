// fwd_f32.hip — float32 forward pass for all window families (VALU, not MFMA).
//
// The float32 I/O path is for callers that need full single precision; it is
// not the performance path.  One wave computes one query row: lanes score 64
// keys of the row's connectivity set at a time (one key per lane), keep an
// online softmax (running max, rescaled sum), and accumulate p*v with each lane
// owning D/64 output columns.
//
// Connectivity sets: causal t-W < s <= t ([KB] §2-§3); Longformer: a global
// row attends every position, any other row attends i + k*dil (|k| <= r) inside
// [0, T) plus the global positions not already in that window ([PP] §1.1,
// §3.1, §4.3); ring: a query at absolute position p attends the ring slots
// holding a position in (p-W, p] ([G3] "How it works").  Causal and ring
// modes take attention sinks: the first n_sink positions stay visible ([KB] §4
// "Failure mode 1"; [ST] "What's New") and a per-head sink score may join the
// denominator.  Dilated causal heads ([KB] §2 "Dilation") attend
// {t - i*d : 0 <= i < W}, cut at 0.  With separate global projections ([PP] §5.2) a global row
// reads q_g against k_g, v_g, and any other row reads every global key through
// k_g, v_g and only the non-global window keys through k, v.  Scores use the
// masked softmax of [KB] §2.
//
// Tags: [KB] knowledge-base page "Sliding Window Attention" (lizeman.github.io);
// [PP] "Sliding Window Attention: From Local Windows to Global Context" (prathamp.com);
// [G3] "Sliding Window Attention — Gemma 3" study note (ai-engineer-exhaustive.pages.dev).

#include "swa_internal.h"

namespace swa {
namespace {

template <int D, int MODE>
__global__ __launch_bounds__(256) void fwd_f32_kernel(const FwdArgs a, const GlobalList gl) {
  constexpr bool GPROJ = MODE == kSymmetricProj;  // separate global projections
  constexpr bool SYM = MODE == kSymmetric || GPROJ;
  constexpr bool RING = MODE == kRing;
  constexpr bool CDIL = MODE == kCausalDil;  // dilated causal: a.dil[h] per query head
  constexpr int DPL = D / 64;  // output columns per lane
  __shared__ float qs[4][D];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const long long row_id = (long long)blockIdx.x * 4 + wave;  // (b, h, t) flattened
  const long long n_rows = (long long)a.B * a.Hq * a.T;
  const bool live = row_id < n_rows;
  const int t = live ? (int)(row_id % a.T) : 0;
  const int h = live ? (int)((row_id / a.T) % a.Hq) : 0;
  const int b = live ? (int)(row_id / ((long long)a.T * a.Hq)) : 0;
  const int kvh = SYM ? h : h / a.group;
  const float *q = static_cast<const float *>(a.q);
  const long long kv_off = (long long)b * a.k_sb + (long long)kvh * a.k_sh;
  const float *k = static_cast<const float *>(a.k) + kv_off;
  const float *v = static_cast<const float *>(a.v) + kv_off;
  // keys and values of global positions (K_g, V_g, or the shared k, v)
  const float *kgl = GPROJ ? static_cast<const float *>(a.kg) + kv_off : k;
  const float *vgl = GPROJ ? static_cast<const float *>(a.vg) + kv_off : v;
  bool is_glob = false;
  if constexpr (SYM)
    for (int g = 0; g < a.G; ++g) is_glob |= live && gl.idx[b * a.G + g] == t;
  // a global row reads its query from Q_g and every key from K_g, V_g
  if (GPROJ && is_glob) {
    q = static_cast<const float *>(a.qg);
    k = kgl;
    v = vgl;
  }
  const float *qrow = q + (long long)b * a.q_sb + (long long)t * a.q_st + (long long)h * D;
  if (!SYM && !RING && a.rope) {
    // rotary positions on the query (rotate-half pairs (i, i + D/2) at position t)
    for (int i = lane; i < D / 2; i += 64) {
      float xa = 0.f, xb = 0.f;
      if (live) {
        xa = qrow[i];
        xb = qrow[i + D / 2];
        const double xr = (double)t * (a.rope_rev0 * rope_pow(a.rope_step, i));
        float sn, cs;
        sincosf((float)((xr - floor(xr)) * 6.283185307179586), &sn, &cs);
        const float ra = xa * cs - xb * sn, rb = xb * cs + xa * sn;
        xa = ra;
        xb = rb;
      }
      qs[wave][i] = xa;
      qs[wave][i + D / 2] = xb;
    }
  } else {
    for (int d = lane; d < D; d += 64) qs[wave][d] = live ? qrow[d] : 0.f;
  }
  __syncthreads();
  if (!live) return;

  // Enumerate the connectivity set as idx -> key position (or -1 = skip); a
  // key at position p read through K_g, V_g is encoded as -2 - p.
  int n_keys, base = 0, kstep = 1, n_win = 0, n_sk = 0;
  const int dil = SYM ? a.dil[h] : 1;
  int my_pos = 0;
  if constexpr (RING) {
    n_keys = a.S;  // every slot; the position test below picks the window
    my_pos = a.q_pos[(long long)b * a.T + t];
  } else if constexpr (CDIL) {
    kstep = a.dil[h];
    n_keys = min(a.W, t / kstep + 1);  // keys t, t - d, ..., >= 0
  } else if constexpr (!SYM) {
    base = max(0, t - a.W + 1);
    n_sk = min(a.n_sink, base);  // sink tokens before the window
    n_keys = n_sk + t - base + 1;
  } else {
    if (is_glob) {
      n_keys = a.T;
    } else {
      const int r = a.W;
      const int k_lo = max(-r, -(t / dil));
      const int k_hi = min(r, (a.T - 1 - t) / dil);
      base = t + k_lo * dil;
      kstep = dil;
      n_win = k_hi - k_lo + 1;
      n_keys = n_win + a.G;
    }
  }

  float m = -INFINITY, l = 0.f, acc[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) acc[i] = 0.f;
  for (int c0 = 0; c0 < n_keys; c0 += 64) {
    const int idx = c0 + lane;
    int key = -1;
    if (idx < n_keys) {
      if constexpr (RING) {
        const int p = a.slot_pos[(long long)b * a.S + idx];
        key = (p >= 0 && p <= my_pos && (p > my_pos - a.W || p < a.n_sink)) ? idx : -1;
      } else if constexpr (CDIL) {
        key = t - idx * kstep;
      } else if constexpr (!SYM) {
        key = (idx < n_sk) ? idx : base + (idx - n_sk);
      } else if (is_glob) key = base + idx * kstep;
      else if (idx < n_win) {
        key = base + idx * kstep;
        if constexpr (GPROJ)  // a global position is read through K_g below
          for (int g = 0; g < a.G; ++g)
            if (gl.idx[b * a.G + g] == key) key = -1;
      } else {
        const int g = gl.idx[b * a.G + idx - n_win];
        if constexpr (GPROJ) key = -2 - g;
        else key = dilated_in(t, g, a.W, dil) ? -1 : g;  // already counted in the window
      }
    }
    float s = -INFINITY;
    if (key >= 0 || key <= -2) {
      const float *kr = key >= 0 ? k + (long long)key * a.k_st : kgl + (long long)(-2 - key) * a.k_st;
      float dot = 0.f;
#pragma unroll 8
      for (int d = 0; d < D; ++d) dot = fmaf(qs[wave][d], kr[d], dot);
      s = dot * a.sl2;  // log2 domain
    }
    float cm = s;
#pragma unroll
    for (int x = 32; x >= 1; x >>= 1) cm = fmaxf(cm, __shfl_xor(cm, x));
    const float m_new = fmaxf(m, cm);
    const float mu = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2f(m - mu);
    const float p = exp2f(s - mu);
    float ps = p;
#pragma unroll
    for (int x = 32; x >= 1; x >>= 1) ps += __shfl_xor(ps, x);
    l = l * alpha + ps;
    m = m_new;
#pragma unroll
    for (int i = 0; i < DPL; ++i) acc[i] *= alpha;
    const int cnt = min(64, n_keys - c0);
    for (int u = 0; u < cnt; ++u) {
      const float pu = __shfl(p, u);
      const int ku = __shfl(key, u);
      if (ku >= 0 || ku <= -2) {
        const float *vr = ku >= 0 ? v + (long long)ku * a.k_st : vgl + (long long)(-2 - ku) * a.k_st;
#pragma unroll
        for (int i = 0; i < DPL; ++i) acc[i] = fmaf(pu, vr[lane + 64 * i], acc[i]);
      }
    }
  }
  float inv = (l > 0.f) ? 1.f / l : 0.f;
  float lse2 = (l > 0.f) ? m + log2f(l) : -INFINITY;  // log2 units
  if (!SYM && !CDIL && a.sink_logit) {
    // the sink score z joins the denominator: 2^(z log2 e - m) against max(m, z)
    const float z2 = a.sink_logit[h] * 1.4426950408889634f;
    const float mu = (m == -INFINITY) ? z2 : fmaxf(m, z2);
    const float sc = (l > 0.f) ? exp2f(m - mu) : 0.f;
    const float lt = l * sc + exp2f(z2 - mu);
    inv = sc / lt;
    lse2 = mu + log2f(lt);
  }
  float *o = static_cast<float *>(a.o) + (long long)b * a.q_sb + (long long)t * a.q_st + (long long)h * D;
#pragma unroll
  for (int i = 0; i < DPL; ++i) o[lane + 64 * i] = acc[i] * inv;
  if (a.lse && lane == 0)
    a.lse[((long long)b * a.Hq + h) * a.T + t] = lse2 * 0.69314718055994531f;
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs &a, int mode, int D, const GlobalList *gl,
                          hipStream_t st) {
  const long long rows = (long long)a.B * a.Hq * a.T;
  const int blocks = (int)((rows + 3) / 4);
  if (blocks <= 0) return hipSuccess;
  const dim3 g(blocks), blk(256);
  if (mode == kCausal || mode == kCausalSink) {  // one kernel; sinks are runtime here
    if (D == 128) hipLaunchKernelGGL((fwd_f32_kernel<128, kCausal>), g, blk, 0, st, a, *gl);
    else hipLaunchKernelGGL((fwd_f32_kernel<64, kCausal>), g, blk, 0, st, a, *gl);
  } else if (mode == kRing) {
    if (D == 128) hipLaunchKernelGGL((fwd_f32_kernel<128, kRing>), g, blk, 0, st, a, *gl);
    else hipLaunchKernelGGL((fwd_f32_kernel<64, kRing>), g, blk, 0, st, a, *gl);
  } else if (mode == kCausalDil) {
    if (D == 128) hipLaunchKernelGGL((fwd_f32_kernel<128, kCausalDil>), g, blk, 0, st, a, *gl);
    else hipLaunchKernelGGL((fwd_f32_kernel<64, kCausalDil>), g, blk, 0, st, a, *gl);
  } else if (mode == kSymmetricProj) {
    if (D == 128) hipLaunchKernelGGL((fwd_f32_kernel<128, kSymmetricProj>), g, blk, 0, st, a, *gl);
    else hipLaunchKernelGGL((fwd_f32_kernel<64, kSymmetricProj>), g, blk, 0, st, a, *gl);
  } else {
    if (D == 128) hipLaunchKernelGGL((fwd_f32_kernel<128, kSymmetric>), g, blk, 0, st, a, *gl);
    else hipLaunchKernelGGL((fwd_f32_kernel<64, kSymmetric>), g, blk, 0, st, a, *gl);
  }
  return hipGetLastError();
}

}  // namespace swa
