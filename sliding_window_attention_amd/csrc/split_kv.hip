// split_kv.hip — few queries against many keys: ring-cache decode and the
// global rows of Longformer attention.
//
// Both are HBM-bound streams over keys.  The keys of one (batch, key/value
// head) are cut into S chunks; each chunk yields, for every query sharing that
// head, the partial softmax state (max m, sum l and the unnormalised sum of
// p*v), and the S partials merge as: with M = max_s m_s, o = sum_s 2^(m_s-M)
// acc_s / sum_s 2^(m_s-M) l_s, which equals the softmax over the union of the
// chunks exactly up to rounding (softmax over a disjoint union).  bf16 decode
// runs the S chunks as the waves of one workgroup and merges them in LDS; the
// other uses give each chunk a workgroup that writes its state to the
// workspace, merged by a second kernel.
//
// Decode mask: slot j is attended iff its stored absolute position p satisfies
// p >= 0 and cur-W < p <= cur ([KB] §2 "KV cache": token p lives in slot p mod W;
// [G3] "How it works": the window comes from stored positions).
// Global rows: a global position attends every position ([PP] §4.3).
//
// Tags: [KB] knowledge-base page "Sliding Window Attention" (lizeman.github.io);
// [G3] "Sliding Window Attention — Gemma 3" study note (ai-engineer-exhaustive);
// [PP] "Sliding Window Attention: From Local Windows to Global Context" (prathamp.com).

#include "swa_internal.h"

namespace swa {
namespace {

constexpr int kMaxQ = 8;        // queries per launch of the split kernel
constexpr int kMaxChunk = 512;  // keys per workgroup

struct alignas(16) U4 {
  uint32_t w[4];
};

// 16 bytes of a key or value row that is read once per call: a non-temporal
// load (the cache lines are marked for early eviction instead of being kept
// for reuse that never comes).  Streaming reads of the ring this way reach
// about 7.0 TB/s on MI355X against about 6.3 TB/s for ordinary loads.
__device__ inline U4 load_stream(const uint16_t *p) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  return __builtin_bit_cast(U4, __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p)));
}

// 8 consecutive elements starting at p, widened to fp32
template <bool F32>
__device__ inline void load8(const void *p, float *out) {
  if constexpr (F32) {
    const float4 a = reinterpret_cast<const float4 *>(p)[0];
    const float4 b = reinterpret_cast<const float4 *>(p)[1];
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
  } else {
    // bf16 -> fp32: the 16 bits become the high half of the fp32 word
    const U4 u = *reinterpret_cast<const U4 *>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(u.w[i] << 16);
      out[2 * i + 1] = __uint_as_float(u.w[i] & 0xffff0000u);
    }
  }
}

template <int D, bool F32, bool DECODE>
__global__ __launch_bounds__(256) void split_kernel(const SplitArgs a, const GlobalList gl, int q_off,
                                                    int nq, int G) {
  constexpr int LPR = D / 8;          // lanes per key row
  constexpr int RPR = 256 / LPR;      // rows per round (whole workgroup)
  constexpr int ES = F32 ? 4 : 2;     // element size
  __shared__ float qs[kMaxQ][D];
  __shared__ float sc[kMaxQ][kMaxChunk];
  __shared__ float red[4][kMaxQ][D];
  __shared__ float ml[kMaxQ][2];
  __shared__ uint8_t key_ok[kMaxChunk];  // key r of the chunk is attended

  const int split = group_x(), kvh = group_y(), b = group_z();
  const int tid = thread_x(), lane = tid & 63, wave = tid >> 6;
  const int c0 = split * a.chunk;
  const int c1 = min(a.n_keys, c0 + a.chunk);
  const int n = c1 - c0;

  // ---- queries -> LDS (fp32)
  for (int i = tid; i < nq * D; i += 256) {
    const int qi = i / D, d = i % D;
    long long off;
    if constexpr (DECODE) off = b * a.q_sb + kvh * a.q_sh + (long long)(q_off + qi) * a.q_sq + d;
    else off = b * a.q_sb + kvh * a.q_sh + (long long)gl.idx[b * G + q_off + qi] * a.q_sq + d;
    float x;
    if constexpr (F32) x = static_cast<const float *>(a.q)[off];
    else x = __uint_as_float((uint32_t) static_cast<const uint16_t *>(a.q)[off] << 16);
    qs[qi][d] = x;
  }
  __syncthreads();

  const char *kb = static_cast<const char *>(a.k) + (b * a.k_sb + kvh * a.k_sh) * ES;
  const char *vb = static_cast<const char *>(a.v) + (b * a.k_sb + kvh * a.k_sh) * ES;
  const int grp = tid / LPR, sub = tid % LPR;  // row group, 8-column chunk
  int cur = 0;
  if constexpr (DECODE) cur = a.cur_pos[b];

  // ---- phase 1: scores (x scale*log2 e); masked keys get -inf
  for (int r0 = 0; r0 < n; r0 += RPR) {
    const int r = r0 + grp;
    float kx[8];
    bool valid = r < n;
    if (valid) load8<F32>(kb + ((c0 + r) * a.k_sr + sub * 8) * ES, kx);
    else
#pragma unroll
      for (int e = 0; e < 8; ++e) kx[e] = 0.f;
    if constexpr (DECODE) {
      if (valid) {
        const int p = a.slot_pos[(long long)b * a.n_keys + c0 + r];
        valid = p >= 0 && p > cur - a.W && p <= cur;
      }
    }
    if (sub == 0 && r < n) key_ok[r] = valid;
    for (int qi = 0; qi < nq; ++qi) {
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) part = fmaf(qs[qi][sub * 8 + e], kx[e], part);
#pragma unroll
      for (int x = 1; x < LPR; x <<= 1) part += __shfl_xor(part, x);
      if (sub == 0 && r < n) sc[qi][r] = valid ? part * a.sl2 : -INFINITY;
    }
  }
  __syncthreads();

  // ---- phase 2: per-query max and sum over the chunk (one wave per query)
  for (int qi = wave; qi < nq; qi += 4) {
    float m = -INFINITY;
    for (int i = lane; i < n; i += 64) m = fmaxf(m, sc[qi][i]);
#pragma unroll
    for (int x = 32; x >= 1; x >>= 1) m = fmaxf(m, __shfl_xor(m, x));
    const float mu = (m == -INFINITY) ? 0.f : m;
    float l = 0.f;
    for (int i = lane; i < n; i += 64) {
      const float p = __builtin_amdgcn_exp2f(sc[qi][i] - mu);
      sc[qi][i] = p;
      l += p;
    }
#pragma unroll
    for (int x = 32; x >= 1; x >>= 1) l += __shfl_xor(l, x);
    if (lane == 0) {
      ml[qi][0] = m;
      ml[qi][1] = l;
    }
  }
  __syncthreads();

  // ---- phase 3: acc[q][d] = sum_r p[q][r] v[r][d]
  float acc[kMaxQ][8];
#pragma unroll
  for (int qi = 0; qi < kMaxQ; ++qi)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[qi][e] = 0.f;
  // keys outside the set are skipped, not multiplied by a zero weight: the
  // value rows of empty or stale ring slots may hold any bits
  for (int r0 = 0; r0 < n; r0 += RPR) {
    const int r = r0 + grp;
    if (r < n && key_ok[r]) {
      float vx[8];
      load8<F32>(vb + ((c0 + r) * a.k_sr + sub * 8) * ES, vx);
#pragma unroll
      for (int qi = 0; qi < kMaxQ; ++qi) {
        if (qi < nq) {
          const float p = sc[qi][r];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[qi][e] = fmaf(p, vx[e], acc[qi][e]);
        }
      }
    }
  }
  // reduce over the row groups of this wave (lanes with equal sub)
#pragma unroll
  for (int qi = 0; qi < kMaxQ; ++qi)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = acc[qi][e];
#pragma unroll
      for (int s = LPR; s < 64; s <<= 1) x += __shfl_xor(x, s);
      acc[qi][e] = x;
    }
  if (lane < LPR)
    for (int qi = 0; qi < nq; ++qi)
#pragma unroll
      for (int e = 0; e < 8; ++e) red[wave][qi][sub * 8 + e] = acc[qi][e];
  __syncthreads();

  // ---- write the partial state: [B][NKV][NQ_total][S] x (D acc, m, l)
  const int nq_tot = a.NQ;
  for (int i = tid; i < nq * D; i += 256) {
    const int qi = i / D, d = i % D;
    const float s = red[0][qi][d] + red[1][qi][d] + red[2][qi][d] + red[3][qi][d];
    const long long slot = (((long long)b * a.NKV + kvh) * nq_tot + q_off + qi) * a.S + split;
    a.ws[slot * (D + 2) + d] = s;
  }
  if (tid < nq) {
    const long long slot = (((long long)b * a.NKV + kvh) * nq_tot + q_off + tid) * a.S + split;
    a.ws[slot * (D + 2) + D] = ml[tid][0];
    a.ws[slot * (D + 2) + D + 1] = ml[tid][1];
  }
}

// One workgroup of D threads per (query, kv head, batch).  The S partial
// states are read in parallel (one split per thread), reduced across the
// workgroup, then every thread merges its output column over all splits.
template <int D>
__device__ inline float block_reduce(float x, bool is_max, float *red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float y = __shfl_xor(x, o);
    x = is_max ? fmaxf(x, y) : x + y;
  }
  if constexpr (D > 64) {
    const int wv = thread_x() >> 6;
    if ((thread_x() & 63) == 0) red[wv] = x;
    __syncthreads();
    x = is_max ? fmaxf(red[0], red[1]) : red[0] + red[1];
    __syncthreads();
  }
  return x;
}

template <int D, bool F32, bool DECODE>
__global__ __launch_bounds__(128) void combine_kernel(const SplitArgs a, const GlobalList gl, int G) {
  __shared__ float red[2];
  const int qi = group_x(), kvh = group_y(), b = group_z();
  const int d = thread_x();
  const long long base = (((long long)b * a.NKV + kvh) * a.NQ + qi) * a.S;
  const float *ws = a.ws + base * (D + 2);
  float m_loc = -INFINITY;
  for (int s = d; s < a.S; s += D) m_loc = fmaxf(m_loc, ws[s * (D + 2) + D]);
  const float M = block_reduce<D>(m_loc, true, red);
  const float Mu = (M == -INFINITY) ? 0.f : M;
  float l_loc = 0.f;
  for (int s = d; s < a.S; s += D)
    l_loc = fmaf(__builtin_amdgcn_exp2f(ws[s * (D + 2) + D] - Mu), ws[s * (D + 2) + D + 1], l_loc);
  const float L = block_reduce<D>(l_loc, false, red);
  float acc = 0.f;
#pragma unroll 8
  for (int s = 0; s < a.S; ++s)
    acc = fmaf(__builtin_amdgcn_exp2f(ws[s * (D + 2) + D] - Mu), ws[s * (D + 2) + d], acc);
  const float out = (L > 0.f) ? acc / L : 0.f;
  long long row;  // output row offset
  if constexpr (DECODE) row = b * a.o_sb + kvh * a.o_sh + (long long)qi * a.o_sq;
  else row = b * a.o_sb + kvh * a.o_sh + (long long)gl.idx[b * G + qi] * a.o_sq;
  if constexpr (F32) static_cast<float *>(a.o)[row + d] = out;
  else {
    const __bf16 h = (__bf16)out;
    static_cast<uint16_t *>(a.o)[row + d] = __builtin_bit_cast(uint16_t, h);
  }
  if (a.lse && d == 0) {
    const float lse = (L > 0.f) ? (M + __log2f(L)) * 0.69314718055994531f : -INFINITY;
    if constexpr (DECODE) a.lse[((long long)b * a.NKV + kvh) * a.NQ + qi] = lse;
    else {
      // lse layout [B][H][T]; n_keys == T for global rows
      a.lse[((long long)b * a.NKV + kvh) * a.n_keys + gl.idx[b * G + qi]] = lse;
    }
  }
}

// ---- bf16 path: one wave per (split, kv head, query pass, batch) ----------------
//
// Keys are walked in blocks of 32.  Per block:
//   S^T = K Q^T on v_mfma_f32_32x32x16_bf16: the A operand (K) is loaded from
//         HBM straight into the operand layout (lane = key row, 16 bytes per
//         k-step), Q^T (B operand) stays in VGPRs; only QG of the 32 query
//         columns are live (the MFMA has ample headroom on an HBM-bound path);
//   online softmax: each lane owns one query column, the block max / sum is a
//         16-register reduction plus one v_permlane32_swap;
//   O += P V on v_dot2_f32_bf16: lanes own 8 output columns of one row group;
//         rows are paired so each lane reads the pair's two P values as one
//         packed dword from LDS.
// The next block's K/V loads are issued before the current block is computed.

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ inline float xhalf_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float xhalf_add(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Sum of x over the lanes that share lane % N (N = 8, 16 or 32): a butterfly
// over lane ^ N, lane ^ 2N, ... with cross-lane VALU moves (DPP rotation by 8
// inside rows of 16 lanes, v_permlane16_swap, v_permlane32_swap) instead of
// LDS-routed shuffles.  Same pairs and order as the shuffle butterfly.
template <int N>
__device__ inline float lane_group_sum(float x) {
  static_assert(N == 8 || N == 16 || N == 32, "butterfly from lane ^ 8, 16 or 32");
  if constexpr (N == 8)
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));
  if constexpr (N <= 16) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  return xhalf_add(x);
}

__device__ inline uint32_t pack2_bf16(float a, float b) {
  bf16x2 v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

template <int D>
struct DecBlock {
  static constexpr int KS = D / 16;    // MFMA k-steps over d_h
  static constexpr int TPR = D / 8;    // lanes per V row (16 bytes each)
  static constexpr int RG = 64 / TPR;  // V row groups per wave
  static constexpr int RPL = 32 / RG;  // V rows per lane per block
  U4 k[KS];
  U4 v[RPL];
  int valid;                           // this lane's key (lane & 31) is attended
};

// The block's key rows, read as whole rows: load i brings rows RG*i .. RG*i +
// RG-1 (TPR lanes per row, 16 bytes each), so every cache line is used up by
// the load that fetches it and the loads can be non-temporal.  kst_to_operand
// then moves them into the MFMA operand layout through the wave's LDS slice.
template <int D>
__device__ inline void dec_load_k(DecBlock<D> &blk, const uint16_t *kbase, const SplitArgs &a,
                                  int s0, int c1, int lane) {
  using Bk = DecBlock<D>;
  static_assert(Bk::RPL == Bk::KS, "one row-group load per MFMA k-step register");
  const int g = lane / Bk::TPR, c = lane % Bk::TPR;
#pragma unroll
  for (int i = 0; i < Bk::RPL; ++i) {
    const int sk = s0 + Bk::RG * i + g;
    if (sk < c1) blk.k[i] = load_stream(kbase + (long long)sk * a.k_sr + c * 8);
    else blk.k[i] = U4{{0, 0, 0, 0}};
  }
}

// 16-byte chunk c of key row r sits at chunk c ^ kst_swz(r) of the row in LDS:
// the operand reads (16 lanes at a time, 16 consecutive rows, one logical
// chunk) then hit 16 distinct bank groups.
template <int D>
__device__ inline int kst_swz(int row) { return D == 128 ? (row & 15) : ((row >> 1) & 7); }

// Key rows from the whole-row layout of dec_load_k to the A-operand layout of
// S^T = K Q^T (lane: key lane & 31, columns 16 ks + 8 (lane >> 5) .. +7), in
// place, through this wave's LDS slice kl (32 rows).  One wave writes and reads
// its own slice; LDS operations of a wave complete in order.  The swizzle of
// row RG i + g is kst_swz(RG i) ^ kst_swz(g) and that of chunk 2 ks + lh is
// (2 ks) ^ lh (disjoint bits), so every offset is one per-lane base XOR a
// constant: two base registers instead of one offset register per load.
template <int D>
__device__ inline void kst_to_operand(DecBlock<D> &blk, char *kl, int lane) {
  using Bk = DecBlock<D>;
  constexpr int ROWB = 2 * D;
  const int g = lane / Bk::TPR, c = lane % Bk::TPR;
  const int lq = lane & 31, lh = lane >> 5;
  int wbase = g * ROWB + ((c ^ kst_swz<D>(g)) * 16);
  int rbase = lq * ROWB + ((lh ^ kst_swz<D>(lq)) * 16);
  // recomputed where used (kept out of loop-invariant registers)
  asm volatile("" : "+v"(wbase), "+v"(rbase));
#pragma unroll
  for (int i = 0; i < Bk::RPL; ++i)
    *reinterpret_cast<U4 *>(kl + ((wbase ^ (kst_swz<D>(Bk::RG * i) * 16)) + i * Bk::RG * ROWB)) = blk.k[i];
#pragma unroll
  for (int ks = 0; ks < Bk::KS; ++ks)
    blk.k[ks] = *reinterpret_cast<const U4 *>(kl + (rbase ^ (32 * ks)));
}

template <int D, bool DECODE>
__device__ inline int dec_valid(const SplitArgs &a, int b, int s0, int c1, int cur, int lane) {
  const int sk = s0 + (lane & 31);
  int ok = sk < c1;
  if constexpr (DECODE) {
    if (ok) {
      const int p = a.slot_pos[(long long)b * a.n_keys + sk];
      ok = p >= 0 && p > cur - a.W && p <= cur;
    }
  }
  return ok;
}

template <int D>
__device__ inline void dec_load_v(DecBlock<D> &blk, const uint16_t *vbase, const SplitArgs &a,
                                  int s0, int c1, int lane) {
  using Bk = DecBlock<D>;
  const int g = lane / Bk::TPR, c = lane % Bk::TPR;
#pragma unroll
  for (int i = 0; i < Bk::RPL; ++i) {
    const int sv = s0 + Bk::RG * i + g;
    if (sv < c1) blk.v[i] = load_stream(vbase + (long long)sv * a.k_sr + c * 8);
    else blk.v[i] = U4{{0, 0, 0, 0}};
  }
}

// NSW = 0: one wave per workgroup, workgroup x = split; the partial states go
// to the workspace for combine_kernel.  NSW >= 1: the workgroup's NSW waves
// are the splits of one (batch, kv head, query pass) and merge their partial
// states in LDS at the end (no workspace, no second kernel).
template <int D, int QG, bool DECODE, int NSW>
__global__ __launch_bounds__(64 * (NSW > 0 ? NSW : 1), QG >= 8 ? 1 : 2) void split_mfma_kernel(
    const SplitArgs a, const GlobalList gl, int G, int n_pass) {
  using Bk = DecBlock<D>;
  constexpr int KS = Bk::KS, TPR = Bk::TPR, RG = Bk::RG, RPL = Bk::RPL;
  constexpr int NPAIR = RPL / 2;
  constexpr int NWG = NSW > 0 ? NSW : 1;  // waves per workgroup
  // [wave][parity][pair][row group][query]
  __shared__ uint32_t ppair_all[NWG][2][NPAIR][RG][QG];
  // each wave's key block on its way to the MFMA operand layout
  __shared__ __attribute__((aligned(16))) char kst_all[NWG][32 * 2 * D];

  const int lane = thread_x() & 63;
  const int wave = __builtin_amdgcn_readfirstlane(thread_x() >> 6);
  const int lq = lane & 31, lh = lane >> 5;
  const int split = NSW > 0 ? wave : group_x();
  auto &ppair = ppair_all[wave];
  const int kvh = group_y() / n_pass, q0 = (group_y() % n_pass) * QG;
  const int b = group_z();
  const int nq = min(QG, a.NQ - q0);
  // Keys of this wave: with NSW = 0 the split's chunk [c0, c1) in 32-key
  // blocks; with NSW > 0 the waves interleave 32-key blocks (wave w takes
  // blocks w, w + NSW, ...), so the workgroup reads K and V as two contiguous
  // streams.  bstep = distance between a wave's consecutive blocks.
  const int c0 = NSW > 0 ? 32 * wave : split * a.chunk;
  const int c1 = NSW > 0 ? a.n_keys : min(a.n_keys, c0 + a.chunk);
  constexpr int bstep = 32 * NWG;
  const int nblk = NSW > 0 ? (c1 > c0 ? (c1 - c0 + bstep - 1) / bstep : 0) : (c1 - c0 + 31) / 32;
  int cur = 0;
  if constexpr (DECODE) cur = a.cur_pos[b];

  // Q^T (B operand): lane holds query lq, columns 16ks + 8lh .. +7
  bf16x8 qf[KS];
  {
    const uint16_t *qg = static_cast<const uint16_t *>(a.q);
    long long row = -1;
    if (lq < nq) {
      if constexpr (DECODE) row = (long long)(q0 + lq) * a.q_sq;
      else row = (long long)gl.idx[b * G + q0 + lq] * a.q_sq;
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      U4 u = U4{{0, 0, 0, 0}};
      if (row >= 0)
        u = *reinterpret_cast<const U4 *>(qg + b * a.q_sb + kvh * a.q_sh + row + ks * 16 + lh * 8);
      qf[ks] = __builtin_bit_cast(bf16x8, u);
    }
  }
  const uint16_t *kbase = static_cast<const uint16_t *>(a.k) + b * a.k_sb + kvh * a.k_sh;
  const uint16_t *vbase = static_cast<const uint16_t *>(a.v) + b * a.k_sb + kvh * a.k_sh;

  float m_run = -INFINITY, l_run = 0.f;
  float acc[QG][8];
#pragma unroll
  for (int q = 0; q < QG; ++q)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[q][e] = 0.f;
  const int g = lane / TPR;

  DecBlock<D> blk;
  if (nblk > 0) {
    dec_load_k<D>(blk, kbase, a, c0, c1, lane);
    dec_load_v<D>(blk, vbase, a, c0, c1, lane);
    blk.valid = dec_valid<D, DECODE>(a, b, c0, c1, cur, lane);
  }
  for (int ib = 0; ib < nblk; ++ib) {
    const int parity = ib & 1;
    const int s_next = c0 + (NSW > 0 ? bstep : 32) * (ib + 1);
    const bool more = ib + 1 < nblk;
    kst_to_operand<D>(blk, kst_all[wave], lane);
    f32x16 s = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, blk.k[ks]), qf[ks], s,
                                                  0, 0, 0);
    // accumulator element j holds key 8(j/4) + 4lh + (j%4) of the block
    const unsigned long long vm = __ballot(lane < 32 && blk.valid);
    // K registers are free again: start the next block's K (and mask) loads
    if (more) {
      dec_load_k<D>(blk, kbase, a, s_next, c1, lane);
      blk.valid = dec_valid<D, DECODE>(a, b, s_next, c1, cur, lane);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int key = 8 * (j >> 2) + 4 * lh + (j & 3);
      if (!((vm >> key) & 1ull)) s[j] = -INFINITY;
      mx = fmaxf(mx, s[j]);
    }
    mx = xhalf_max(mx);
    const float m_new = fmaxf(m_run, mx * a.sl2);
    const float mu = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - mu);
#pragma unroll
    for (int j = 0; j < 16; ++j) s[j] = __builtin_amdgcn_exp2f(fmaf(s[j], a.sl2, -mu));
    // P -> bf16 (RNE), rows paired as (key, key + 8): both live in this lane
    // as elements j and j + 4.  The row sum is taken over these rounded
    // weights (v_dot2 against ones, fp32), the ones the product uses.
    uint32_t pk[8];
    float rs = 0.f;
    const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if ((j & 4) == 0) {
        const int u = (j >> 3) * 4 + (j & 3);
        pk[u] = pack2_bf16(s[j], s[j + 4]);
        rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[u]), ones, rs, false);
      }
    }
    l_run = fmaf(l_run, alpha, xhalf_add(rs));
    m_run = m_new;
    // P pairs -> LDS
    if (lq < QG) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if ((j & 4) == 0) {
          int pi, rg;
          if constexpr (D == 128) {  // row = 4i + rg, i = 2(j/4) + lh, pairs (i, i+2)
            pi = (j >> 3) * 2 + lh;
            rg = j & 3;
          } else {                   // row = 8i + rg, i = j/4, pairs (i, i+1)
            pi = j >> 3;
            rg = 4 * lh + (j & 3);
          }
          ppair[parity][pi][rg][lq] = pk[(j >> 3) * 4 + (j & 3)];
        }
      }
    }
    // every lane reads the P values other lanes of this wave just wrote: LDS
    // operations of one wave complete in order, so waiting for this wave's
    // writes is enough (the other waves of the workgroup use their own slice)
    if constexpr (NSW > 0) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_wave_barrier();
    } else {
      __syncthreads();
    }
#pragma unroll
    for (int q = 0; q < QG; ++q) {
      // alpha of query q lives in lane q
      const float aq = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(alpha), q));
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[q][e] *= aq;
    }
#pragma unroll
    for (int pi = 0; pi < NPAIR; ++pi) {
      int i0, i1;
      if constexpr (D == 128) {
        i0 = (pi >> 1) * 4 + (pi & 1);
        i1 = i0 + 2;
      } else {
        i0 = 2 * pi;
        i1 = i0 + 1;
      }
      // value rows of keys outside the set (empty, stale or future slots, or
      // past the end) are zeroed: their weight is 0, but 0 times the NaN or
      // Inf bits an unwritten slot may hold would not be
      const uint32_t z0 = ((vm >> (RG * i0 + g)) & 1ull) ? 0xffffffffu : 0u;
      const uint32_t z1 = ((vm >> (RG * i1 + g)) & 1ull) ? 0xffffffffu : 0u;
      uint32_t w[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t x0 = blk.v[i0].w[e] & z0, x1 = blk.v[i1].w[e] & z1;
        w[2 * e] = (x0 & 0xffffu) | (x1 << 16);
        w[2 * e + 1] = (x0 >> 16) | (x1 & 0xffff0000u);
      }
#pragma unroll
      for (int q = 0; q < QG; ++q) {
        const uint32_t pp = ppair[parity][pi][g][q];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          acc[q][e] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pp),
                                                      __builtin_bit_cast(bf16x2, w[e]), acc[q][e],
                                                      false);
      }
    }
    // V registers are free again: start the next block's V loads
    if (more) dec_load_v<D>(blk, vbase, a, s_next, c1, lane);
  }

  // reduce acc over the row groups (lanes with equal lane % TPR)
#pragma unroll
  for (int q = 0; q < QG; ++q)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      acc[q][e] = lane_group_sum<TPR>(acc[q][e]);
    }
  const long long base = ((long long)b * a.NKV + kvh) * a.NQ;
  if constexpr (NSW == 0) {
    if (lane < TPR) {
#pragma unroll
      for (int q = 0; q < QG; ++q) {
        if (q < nq) {
          float *dst = a.ws + ((base + q0 + q) * a.S + split) * (D + 2) + lane * 8;
#pragma unroll
          for (int e = 0; e < 8; ++e) dst[e] = acc[q][e];
        }
      }
    }
    if (lh == 0 && lq < nq) {
      float *dst = a.ws + ((base + q0 + lq) * a.S + split) * (D + 2);
      dst[D] = m_run;
      dst[D + 1] = l_run;
    }
  } else {
    // Merge the NSW partial states of the workgroup, exactly as combine_kernel
    // does across workgroups: with M = max_w m_w (log2 units),
    // o = sum_w 2^(m_w - M) acc_w / sum_w 2^(m_w - M) l_w.
    __shared__ float m_acc[NSW][QG][D];
    __shared__ float m_ml[NSW][QG][2];
    if (lane < TPR) {
#pragma unroll
      for (int q = 0; q < QG; ++q)
#pragma unroll
        for (int e = 0; e < 8; ++e) m_acc[wave][q][lane * 8 + e] = acc[q][e];
    }
    if (lh == 0 && lq < QG) {
      m_ml[wave][lq][0] = m_run;
      m_ml[wave][lq][1] = l_run;
    }
    __syncthreads();
    for (int i = thread_x(); i < QG * D; i += 64 * NSW) {
      const int q = i / D, d = i % D;
      if (q >= nq) continue;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < NSW; ++w) M = fmaxf(M, m_ml[w][q][0]);
      const float Mu = (M == -INFINITY) ? 0.f : M;
      float L = 0.f, o = 0.f;
#pragma unroll
      for (int w = 0; w < NSW; ++w) {
        const float sc = __builtin_amdgcn_exp2f(m_ml[w][q][0] - Mu);
        L = fmaf(sc, m_ml[w][q][1], L);
        o = fmaf(sc, m_acc[w][q][d], o);
      }
      o = (L > 0.f) ? o / L : 0.f;
      long long row;
      if constexpr (DECODE) row = b * a.o_sb + kvh * a.o_sh + (long long)(q0 + q) * a.o_sq;
      else row = b * a.o_sb + kvh * a.o_sh + (long long)gl.idx[b * G + q0 + q] * a.o_sq;
      const __bf16 hv = (__bf16)o;
      static_cast<uint16_t *>(a.o)[row + d] = __builtin_bit_cast(uint16_t, hv);
      if (a.lse && d == 0) {
        const float lse = (L > 0.f) ? (M + __log2f(L)) * 0.69314718055994531f : -INFINITY;
        if constexpr (DECODE) a.lse[base + q0 + q] = lse;
        else a.lse[((long long)b * a.NKV + kvh) * a.n_keys + gl.idx[b * G + q0 + q]] = lse;
      }
    }
  }
}

template <int D, int QG, bool DECODE>
void launch_mfma_qg(const SplitArgs &a, const GlobalList *gl, int G, int n_pass, int nsw,
                    hipStream_t st) {
  if (nsw == 0) {
    hipLaunchKernelGGL((split_mfma_kernel<D, QG, DECODE, 0>), dim3(a.S, a.NKV * n_pass, a.B),
                       dim3(64), 0, st, a, *gl, G, n_pass);
    return;
  }
  const dim3 grid(1, a.NKV * n_pass, a.B);
  switch (nsw) {
    case 1: hipLaunchKernelGGL((split_mfma_kernel<D, QG, DECODE, 1>), grid, dim3(64), 0, st, a, *gl, G, n_pass); break;
    case 2: hipLaunchKernelGGL((split_mfma_kernel<D, QG, DECODE, 2>), grid, dim3(128), 0, st, a, *gl, G, n_pass); break;
    case 4: hipLaunchKernelGGL((split_mfma_kernel<D, QG, DECODE, 4>), grid, dim3(256), 0, st, a, *gl, G, n_pass); break;
    default: hipLaunchKernelGGL((split_mfma_kernel<D, QG, DECODE, 8>), grid, dim3(512), 0, st, a, *gl, G, n_pass); break;
  }
}

template <int D, bool DECODE>
hipError_t run_mfma(const SplitArgs &a, const GlobalList *gl, int G, hipStream_t st) {
  const int qg = mfma_qg(a.NQ);
  const int n_pass = (a.NQ + qg - 1) / qg;
  // a.S in {1, 2, 4, 8} with a.merge set: the splits are the waves of one
  // workgroup and merge in LDS; otherwise one workgroup per split + combine
  const int nsw = a.merge ? a.S : 0;
  switch (qg) {
    case 8: launch_mfma_qg<D, 8, DECODE>(a, gl, G, n_pass, nsw, st); break;
    case 4: launch_mfma_qg<D, 4, DECODE>(a, gl, G, n_pass, nsw, st); break;
    case 2: launch_mfma_qg<D, 2, DECODE>(a, gl, G, n_pass, nsw, st); break;
    default: launch_mfma_qg<D, 1, DECODE>(a, gl, G, n_pass, nsw, st); break;
  }
  if (a.merge) return hipGetLastError();
  hipLaunchKernelGGL((combine_kernel<D, false, DECODE>), dim3(a.NQ, a.NKV, a.B), dim3(D), 0, st, a,
                     *gl, G);
  return hipGetLastError();
}

template <int D, bool F32, bool DECODE>
hipError_t run(const SplitArgs &a, const GlobalList *gl, int G, hipStream_t st) {
  dim3 grid(a.S, a.NKV, a.B);
  for (int q0 = 0; q0 < a.NQ; q0 += kMaxQ) {
    const int nq = min(kMaxQ, a.NQ - q0);
    hipLaunchKernelGGL((split_kernel<D, F32, DECODE>), grid, dim3(256), 0, st, a, *gl, q0, nq, G);
  }
  hipLaunchKernelGGL((combine_kernel<D, F32, DECODE>), dim3(a.NQ, a.NKV, a.B), dim3(D), 0, st, a,
                     *gl, G);
  return hipGetLastError();
}

// Ring append ([KB] §2 "KV cache": token i lives in slot i mod S; the slot
// records its absolute position, [G3] "How it works").  With n_sink pinned sink
// tokens ([KB] §4 "Failure mode 1") positions below n_sink keep their own slots
// and the rest roll over the remaining S - n_sink.  Block (hk, t, b) copies
// token t's key and value rows of head hk; the chunk's slots are distinct (a
// documented precondition), so blocks never write the same slot.
__global__ void cache_write_kernel(const char *kn, const char *vn, const int *pos, char *kc,
                                   char *vc, int *slot_pos, int L, int S, int Hkv, int row_bytes,
                                   int n_sink) {
  const int hk = group_x(), t = group_y(), b = group_z();
  const int p = pos[(long long)b * L + t];
  if (p < 0) return;  // documented precondition; never index with a negative slot
  // sink tokens (p < n_sink) keep slot p; the rest roll over the other slots
  const int slot = (p < n_sink) ? p : n_sink + (p - n_sink) % (S - n_sink);
  const long long src = (((long long)b * L + t) * Hkv + hk) * row_bytes;
  const long long dst = (((long long)b * Hkv + hk) * S + slot) * row_bytes;
  for (int i = thread_x() * 4; i < row_bytes; i += group_size_x() * 4) {
    *reinterpret_cast<uint32_t *>(kc + dst + i) = *reinterpret_cast<const uint32_t *>(kn + src + i);
    *reinterpret_cast<uint32_t *>(vc + dst + i) = *reinterpret_cast<const uint32_t *>(vn + src + i);
  }
  if (hk == 0 && thread_x() == 0) slot_pos[(long long)b * S + slot] = p;
}

__global__ void debug_mask_kernel(int mode, int T, int w_or_r, int dil, const GlobalList gl, int G,
                                  uint8_t *mask) {
  const long long i = group_x() * (long long)group_size_x() + thread_x();
  if (i >= (long long)T * T) return;
  const int t = (int)(i / T), s = (int)(i % T);
  // the row's key bounds of the banded kernels (row_key_bounds), in the
  // residue-class index space they run in
  bool on;
  int lo, hi;
  if (mode == SWA_MODE_CAUSAL) {
    row_key_bounds(false, t, w_or_r, T, &lo, &hi);
    on = s >= lo && s <= hi;
  } else {
    bool t_glob = false, s_glob = false;
    for (int g = 0; g < G; ++g) {
      t_glob |= gl.idx[g] == t;
      s_glob |= gl.idx[g] == s;
    }
    const int rho = t % dil;
    const int n_cls = class_len(class_split(T, dil), rho);
    row_key_bounds(true, t / dil, w_or_r, n_cls, &lo, &hi);
    const bool win = s % dil == rho && s / dil >= lo && s / dil <= hi;
    on = t_glob || s_glob || win;
  }
  mask[i] = on ? 1 : 0;
}

}  // namespace

hipError_t launch_split(const SplitArgs &a, bool decode, bool f32, int D, const GlobalList *gl,
                        int G, int H, hipStream_t st) {
  (void)H;
  if (decode) {
    if (f32) return D == 128 ? run<128, true, true>(a, gl, G, st) : run<64, true, true>(a, gl, G, st);
    return D == 128 ? run_mfma<128, true>(a, gl, G, st) : run_mfma<64, true>(a, gl, G, st);
  }
  if (f32) return D == 128 ? run<128, true, false>(a, gl, G, st) : run<64, true, false>(a, gl, G, st);
  return D == 128 ? run_mfma<128, false>(a, gl, G, st) : run_mfma<64, false>(a, gl, G, st);
}

int split_max_chunk() { return kMaxChunk; }

// Queries per pass of the bf16 split kernel (the query heads sharing a K/V head).
int mfma_qg(int nq) { return nq >= 8 ? 8 : nq >= 4 ? 4 : nq >= 2 ? 2 : 1; }

hipError_t launch_cache_write(bool f32, const void *kn, const void *vn, const int *pos, void *kc,
                              void *vc, int *slot_pos, int B, int L, int S, int Hkv, int D,
                              int n_sink, hipStream_t st) {
  const int row_bytes = D * (f32 ? 4 : 2);
  hipLaunchKernelGGL(cache_write_kernel, dim3(Hkv, L, B), dim3(64), 0, st,
                     static_cast<const char *>(kn), static_cast<const char *>(vn), pos,
                     static_cast<char *>(kc), static_cast<char *>(vc), slot_pos, L, S, Hkv,
                     row_bytes, n_sink);
  return hipGetLastError();
}

hipError_t launch_debug_mask(int mode, int T, int w_or_r, int dil, const GlobalList *gl, int G,
                             uint8_t *mask, hipStream_t st) {
  const long long n = (long long)T * T;
  const int blocks = (int)((n + 255) / 256);
  hipLaunchKernelGGL(debug_mask_kernel, dim3(blocks), dim3(256), 0, st, mode, T, w_or_r, dil, *gl,
                     G, mask);
  return hipGetLastError();
}

}  // namespace swa
