// fwd_bf16.hip — banded attention forward on bf16 MFMA for gfx950.
//
// One workgroup (4 waves) owns one query tile and visits only the key tiles
// that intersect the band ([PP] §6.1/§6.3: only banded entries are computed;
// [ST] "The Mechanism": out-of-window key/value blocks are skipped).  Each
// wave owns 32 query rows of one head.  Per key tile of 64 columns:
//
//   S^T = K Q^T      v_mfma_f32_32x32x16_bf16, K from LDS (A), Q in VGPRs (B)
//   mask             only on tiles the schedule marks as partial
//   online softmax   each lane owns one query row: the row max / sum over the
//                    32x32 accumulator is a 16-register reduction plus one
//                    v_permlane32_swap with the partner half-wave
//   O^T += V^T P^T   P^T stays in VGPRs as the B operand; V^T comes from LDS,
//                    transposed while staging the tile
//
// The score definition is the masked softmax of [KB] §2 (alpha^SWA, o^SWA);
// windows: causal t-W < s <= t ([KB] §2-§3), or, in symmetric mode, the
// undilated window |i-j| <= r inside one residue class of a dilated head plus
// the global keys not already in the window ([PP] §1.1, §3.1, §4.3).
//
// Tags: [KB] knowledge-base page "Sliding Window Attention" (lizeman.github.io);
// [PP] "Sliding Window Attention: From Local Windows to Global Context"
// (prathamp.com); [ST] "Sliding Window Attention (SWA)" glossary (superteams.ai).

#include "swa_internal.h"

namespace swa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

struct alignas(16) U4 {
  uint32_t w[4];
};

__device__ inline bf16x8 as_bf16x8(U4 u) { return __builtin_bit_cast(bf16x8, u); }

__device__ inline uint32_t pack_bf16(float a, float b) {
  // v_cvt_pk_bf16_f32: round-to-nearest-even on both halves
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// Partner value of lane l^32 combined with max / add.
__device__ inline float xhalf_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float xhalf_add(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---- LDS layouts ---------------------------------------------------------------
// K tile: [64 keys][D] bf16; the 16-byte chunk c of key row s sits at chunk
// c ^ (s & 7), so the 8 lanes of an MFMA operand read (8 rows, same chunk)
// touch 8 distinct bank groups.
template <int D>
__device__ inline int k_off(int key, int chunk) {
  return key * D + ((chunk ^ (key & 7)) << 3);
}
// V^T tile: [D][64 key positions] bf16.  Keys are permuted inside each group
// of 16 (bits 2 and 3 swapped) so that the 8 keys one lane feeds to the PV
// MFMA are contiguous, and chunks are XOR-swizzled by (d ^ d>>3) & 7 so both
// the operand reads (consecutive d) and the staging writes (d spaced by 8)
// spread over the banks.
__device__ inline int vpos(int key) {
  return (key & ~15) | (key & 3) | ((key & 4) << 1) | ((key & 8) >> 1);
}
__device__ inline int vt_off(int d, int pos) {
  return d * kBN + ((((pos >> 3) ^ ((d ^ (d >> 3)) & 7))) << 3) + (pos & 7);
}

template <int D>
struct Smem {
  static constexpr int kTile = kBN * D;           // elements per K (or V^T) tile
  uint16_t kv[2][2][kTile];                        // [buffer][K, V^T]
};

// ---- per-tile staging ------------------------------------------------------------
// Thread t loads KPT consecutive key rows x 8 columns (16 bytes each), so the
// V^T store can pack KPT keys per column.  Rows of one wave-instruction are
// full contiguous d_h-wide rows (coalesced).
template <int D>
struct Stage {
  static constexpr int TPR = D / 8;          // threads per row
  static constexpr int KPT = kBN * TPR / 256; // keys per thread (4 for D=128, 2 for D=64)
  U4 k[KPT], v[KPT];
};

template <int D>
__device__ inline void stage_load(Stage<D> &st, const uint16_t *kbase, const uint16_t *vbase,
                                  const long long *row_off, int tid) {
  constexpr int TPR = Stage<D>::TPR, KPT = Stage<D>::KPT;
  const int chunk = tid % TPR;
#pragma unroll
  for (int r = 0; r < KPT; ++r) {
    const long long off = row_off[r];
    if (off >= 0) {
      st.k[r] = *reinterpret_cast<const U4 *>(kbase + off + chunk * 8);
      st.v[r] = *reinterpret_cast<const U4 *>(vbase + off + chunk * 8);
    } else {
      st.k[r] = U4{{0, 0, 0, 0}};
      st.v[r] = U4{{0, 0, 0, 0}};
    }
  }
}

template <int D>
__device__ inline void stage_store(const Stage<D> &st, uint16_t *ks, uint16_t *vts, int tid) {
  constexpr int TPR = Stage<D>::TPR, KPT = Stage<D>::KPT;
  const int chunk = tid % TPR;
  const int key0 = KPT * (tid / TPR);
#pragma unroll
  for (int r = 0; r < KPT; ++r)
    *reinterpret_cast<U4 *>(ks + k_off<D>(key0 + r, chunk)) = st.k[r];
  const int p = vpos(key0);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int d = chunk * 8 + e;
    const int word = e >> 1, hi = e & 1;
    uint32_t h[KPT];
#pragma unroll
    for (int r = 0; r < KPT; ++r) h[r] = hi ? (st.v[r].w[word] >> 16) : (st.v[r].w[word] & 0xffffu);
    if constexpr (KPT == 4) {
      uint2 out;
      out.x = h[0] | (h[1] << 16);
      out.y = h[2] | (h[3] << 16);
      *reinterpret_cast<uint2 *>(vts + vt_off(d, p)) = out;
    } else {
      *reinterpret_cast<uint32_t *>(vts + vt_off(d, p)) = h[0] | (h[1] << 16);
    }
  }
}

// ---- the kernel ------------------------------------------------------------------

template <int D, bool SYM>
__global__ __launch_bounds__(256, 2) void fwd_kernel(const FwdArgs a, const GlobalList gl) {
  __shared__ Smem<D> sm;
  constexpr int KS_QK = D / 16;  // k-steps of S = Q K^T
  constexpr int DB = D / 32;     // 32-wide d blocks of O^T
  constexpr int KPT = Stage<D>::KPT, TPR = Stage<D>::TPR;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lq = lane & 31, lh = lane >> 5;

  // -------- work decode
  int b, h, kvh, row0;  // row0: first query row (class index in symmetric mode)
  int rho = 0, dil = 1, n_cls;  // residue class, dilation, class length
  int tile_row0, tile_rows;     // workgroup's query rows (for the tile schedule)
  if constexpr (!SYM) {
    const int nblk = a.B * a.n_hg * a.n_qt;
    const int lid = xcd_remap(blockIdx.x, nblk);
    const int qt = a.n_qt - 1 - (lid % a.n_qt);  // heavy (full-band) tiles first
    const int rest = lid / a.n_qt;
    const int hg = rest % a.n_hg;
    b = rest / a.n_hg;
    h = hg * a.P + (wave % a.P);
    kvh = h / a.group;
    tile_row0 = qt * a.BM;
    row0 = tile_row0 + (wave / a.P) * kRowsPerWave;
    n_cls = a.T;
  } else {
    const int nblk = a.B * a.tiles_per_batch;
    const int lid = xcd_remap(blockIdx.x, nblk);
    b = lid / a.tiles_per_batch;
    const int rem = lid % a.tiles_per_batch;
    int lo = 0, hi = a.Hq - 1;  // find head: head_off[h] <= rem < head_off[h+1]
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.head_off[mid] <= rem) lo = mid; else hi = mid - 1;
    }
    h = lo;
    kvh = h;
    dil = a.dil[h];
    int tile;
    class_tile_decode(a.T, dil, a.BM, rem - a.head_off[h], &rho, &tile);
    n_cls = class_len(class_split(a.T, dil), rho);
    tile_row0 = tile * a.BM;
    row0 = tile_row0 + wave * kRowsPerWave;
  }
  const int t1_valid = min(tile_row0 + a.BM, n_cls) - 1;  // last valid row of the tile

  const uint16_t *qg = static_cast<const uint16_t *>(a.q);
  const uint16_t *kg = static_cast<const uint16_t *>(a.k);
  const uint16_t *vg = static_cast<const uint16_t *>(a.v);
  // position of class row i: rho + dil*i (dil = 1, rho = 0 in causal mode)
  const long long q_rowstride = a.q_st * dil;
  const long long k_rowstride = a.k_st * dil;
  const long long k_rho = (long long)rho * a.k_st;
  const uint16_t *kbase = kg + (long long)b * a.k_sb + (long long)kvh * D;
  const uint16_t *vbase = vg + (long long)b * a.k_sb + (long long)kvh * D;

  // -------- Q (B operand of S^T = K Q^T): lane holds row lq, columns 16ks + 8lh .. +7
  bf16x8 qf[KS_QK];
  {
    const int r = row0 + lq;
    const uint16_t *qp = qg + (long long)b * a.q_sb + (long long)h * D +
                         (long long)rho * a.q_st + (long long)r * q_rowstride;
#pragma unroll
    for (int ks = 0; ks < KS_QK; ++ks) {
      U4 u = U4{{0, 0, 0, 0}};
      if (r < n_cls) u = *reinterpret_cast<const U4 *>(qp + ks * 16 + lh * 8);
      qf[ks] = as_bf16x8(u);
    }
  }

  // -------- schedule
  TileRange tr;
  if constexpr (!SYM) tr = causal_tile_range(tile_row0, t1_valid, a.W, kBN);
  else tr = sym_tile_range(tile_row0, t1_valid, a.W, n_cls, kBN);
  const int n_win = tr.hi - tr.lo + 1;
  const int n_glob = SYM ? ceil_div(a.G, kBN) : 0;
  const int n_tiles = n_win + n_glob;

  // rows this thread stages for tile j (element offsets from kbase; -1 = zero fill)
  auto rows_for = [&](int j, long long *off) {
    const int key0 = KPT * (tid / TPR);
    if (j < n_win) {
      const int s0 = (tr.lo + j) * kBN + key0;
#pragma unroll
      for (int r = 0; r < KPT; ++r)
        off[r] = (s0 + r < n_cls) ? k_rho + (long long)(s0 + r) * k_rowstride : -1;
    } else {
      const int u0 = (j - n_win) * kBN + key0;
#pragma unroll
      for (int r = 0; r < KPT; ++r) {
        // global keys are absolute positions
        off[r] = (u0 + r < a.G) ? (long long)gl.idx[b * a.G + u0 + r] * a.k_st : -1;
      }
    }
  };

  // -------- running softmax state (lane owns query row lq; both half-waves agree)
  f32x16 acc_o[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) acc_o[i] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const int my_row = row0 + lq;

  Stage<D> st;
  {
    long long off[KPT];
    rows_for(0, off);
    stage_load<D>(st, kbase, vbase, off, tid);
    stage_store<D>(st, sm.kv[0][0], sm.kv[0][1], tid);
  }
  __syncthreads();

  for (int j = 0; j < n_tiles; ++j) {
    const int buf = j & 1;
    const bool has_next = j + 1 < n_tiles;
    if (has_next) {
      long long off[KPT];
      rows_for(j + 1, off);
      stage_load<D>(st, kbase, vbase, off, tid);
    }
    const uint16_t *ks = sm.kv[buf][0];
    const uint16_t *vts = sm.kv[buf][1];

    // ---- S^T = K Q^T : two 32-key blocks
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
      const int key = kb * 32 + lq;
#pragma unroll
      for (int kk = 0; kk < KS_QK; ++kk) {
        const U4 u = *reinterpret_cast<const U4 *>(ks + k_off<D>(key, 2 * kk + lh));
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(u), qf[kk], s[kb], 0, 0, 0);
      }
    }

    // ---- mask (partial tiles only).  Accumulator element (kb, e) holds key
    // 32kb + 8(e/4) + 4lh + (e%4) of the tile, for query row my_row.
    bool full;
    int key_base;
    if (j < n_win) {
      const int kj = tr.lo + j;
      key_base = kj * kBN;
      if constexpr (!SYM) full = causal_tile_full(tile_row0, t1_valid, kj, kBN, a.W, n_cls);
      else full = sym_tile_full(tile_row0, t1_valid, kj, kBN, a.W, n_cls);
    } else {
      key_base = (j - n_win) * kBN;
      full = false;
    }
    if (!full) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int kk = key_base + kb * 32 + 8 * (e >> 2) + 4 * lh + (e & 3);
          bool ok;
          if (j < n_win) {
            if constexpr (!SYM) ok = causal_in(my_row, kk, a.W) && kk < n_cls;
            else ok = sym_in(my_row, kk, a.W) && kk < n_cls;
          } else {
            // global key u = kk: attended unless already inside this row's window
            ok = false;
            if (kk < a.G) {
              const int g = gl.idx[b * a.G + kk];
              const int i_abs = rho + dil * my_row;
              ok = !dilated_in(i_abs, g, a.W, dil);
            }
          }
          if (!ok) s[kb][e] = -INFINITY;
        }
    }

    // ---- online softmax in the log2 domain (sl2 = scale * log2 e)
    float mx = s[0][0];
#pragma unroll
    for (int e = 1; e < 16; ++e) mx = fmaxf(mx, s[0][e]);
#pragma unroll
    for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[1][e]);
    mx = xhalf_max(mx);
    const float m_new = fmaxf(m_run, mx * a.sl2);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][e], a.sl2, -m_use));
        s[kb][e] = p;
        rs += p;
      }
    rs = xhalf_add(rs);
    l_run = fmaf(l_run, alpha, rs);
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < DB; ++i) acc_o[i] *= alpha;

    // ---- O^T += V^T P^T : 4 key steps of 16
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int kb = kk >> 1, e0 = (kk & 1) * 8;
      U4 pu;
      pu.w[0] = pack_bf16(s[kb][e0 + 0], s[kb][e0 + 1]);
      pu.w[1] = pack_bf16(s[kb][e0 + 2], s[kb][e0 + 3]);
      pu.w[2] = pack_bf16(s[kb][e0 + 4], s[kb][e0 + 5]);
      pu.w[3] = pack_bf16(s[kb][e0 + 6], s[kb][e0 + 7]);
      const bf16x8 pb = as_bf16x8(pu);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const U4 u = *reinterpret_cast<const U4 *>(vts + vt_off(db * 32 + lq, kk * 16 + lh * 8));
        acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(u), pb, acc_o[db], 0, 0, 0);
      }
    }

    if (has_next) stage_store<D>(st, sm.kv[buf ^ 1][0], sm.kv[buf ^ 1][1], tid);
    __syncthreads();
  }

  // -------- epilogue: normalise, stage rows through LDS, coalesced stores
  const float inv_l = (l_run > 0.f) ? 1.f / l_run : 0.f;
  constexpr int OP = D + 8;  // staging pitch (elements)
  uint16_t *ost = &sm.kv[0][0][0] + wave * (kRowsPerWave * OP);
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d = db * 32 + 8 * g4 + 4 * lh;
      uint2 w;
      w.x = pack_bf16(acc_o[db][4 * g4 + 0] * inv_l, acc_o[db][4 * g4 + 1] * inv_l);
      w.y = pack_bf16(acc_o[db][4 * g4 + 2] * inv_l, acc_o[db][4 * g4 + 3] * inv_l);
      *reinterpret_cast<uint2 *>(ost + lq * OP + d) = w;
    }
  if (a.lse && lh == 0 && my_row < n_cls) {
    const long long t_abs = rho + (long long)dil * my_row;
    const float lse = (l_run > 0.f) ? (m_run + __log2f(l_run)) * 0.69314718055994531f : -INFINITY;
    a.lse[((long long)b * a.Hq + h) * a.T + t_abs] = lse;
  }
  __syncthreads();
  uint16_t *og = static_cast<uint16_t *>(a.o);
  constexpr int LPR = D / 8;             // lanes per row (16 B each)
  constexpr int RPI = 64 / LPR;          // rows per wave instruction
#pragma unroll
  for (int it = 0; it < kRowsPerWave / RPI; ++it) {
    const int rr = it * RPI + lane / LPR;
    const int c = lane % LPR;
    const int r = row0 + rr;
    if (r < n_cls) {
      const U4 u = *reinterpret_cast<const U4 *>(ost + rr * OP + c * 8);
      const long long t_abs = rho + (long long)dil * r;
      *reinterpret_cast<U4 *>(og + (long long)b * a.q_sb + t_abs * a.q_st + (long long)h * D + c * 8) = u;
    }
  }
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs &a, bool symmetric, int D, const GlobalList *gl,
                           hipStream_t st) {
  const int nblk = symmetric ? a.B * a.tiles_per_batch : a.B * a.n_hg * a.n_qt;
  if (nblk <= 0) return hipSuccess;
  dim3 grid(nblk), block(256);
  if (!symmetric) {
    if (D == 128) hipLaunchKernelGGL((fwd_kernel<128, false>), grid, block, 0, st, a, *gl);
    else hipLaunchKernelGGL((fwd_kernel<64, false>), grid, block, 0, st, a, *gl);
  } else {
    if (D == 128) hipLaunchKernelGGL((fwd_kernel<128, true>), grid, block, 0, st, a, *gl);
    else hipLaunchKernelGGL((fwd_kernel<64, true>), grid, block, 0, st, a, *gl);
  }
  return hipGetLastError();
}

}  // namespace swa
