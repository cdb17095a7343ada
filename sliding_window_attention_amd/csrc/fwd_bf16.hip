// fwd_bf16.hip — banded attention forward on bf16 MFMA for gfx950.
//
// One workgroup owns one query tile and visits only the key tiles that
// intersect the band ([PP] §6.1/§6.3: only banded entries are computed; [ST]
// "The Mechanism": out-of-window key/value blocks are skipped).  Each wave owns
// 32 query rows of one head; the waves of a workgroup share one key/value head
// (P query heads x NW/P row blocks), so every staged K/V tile feeds NW waves.
// A wave skips the staged tiles outside its own rows' band.  Key tiles are 32
// keys at d_h = 128 and 64 at d_h = 64; per 32-key block of a tile:
//
//   S^T = K Q^T      v_mfma_f32_32x32x16_bf16, K from LDS (A), Q in VGPRs (B)
//   mask             only on tiles the schedule marks as partial
//   online softmax   each lane owns one query row: the row max over the
//                    32x32 accumulator is a 16-register reduction plus one
//                    v_permlane32_swap with the partner half-wave; the row
//                    sum stays split between the two half-waves (v_dot2 of
//                    the packed P against ones) until the epilogue
//   O^T += V^T P^T   P^T stays in VGPRs as the B operand; the V^T operand is
//                    read from the row-major V tile with ds_read_b64_tr_b16
//
// K and V tiles go from HBM to LDS with global_load_lds_dwordx4 (no VGPR
// staging), double-buffered: tile j+1 is in flight while tile j is computed.
// Each 16-byte chunk of a tile row is XOR-swizzled by the row index so both the
// K operand reads and the transposing V reads hit distinct LDS banks.
//
// The score definition is the masked softmax of [KB] §2 (alpha^SWA, o^SWA);
// windows: causal t-W < s <= t ([KB] §2-§3); in symmetric mode, the
// undilated window |i-j| <= r inside one residue class of a dilated head plus
// the global keys, each key once ([PP] §1.1, §3.1, §4.3); in ring
// mode, a chunk of queries with absolute positions against the slots of a ring
// cache, slot attended iff its stored position p has q_pos-W < p <= q_pos
// ([G3] "How it works": the window comes from positions, not buffer offsets).
// Dilated causal heads ([KB] §2 "Dilation": window {t - i*d : 0 <= i < W})
// run the causal window inside each residue class t mod d, as symmetric mode
// does for dilated Longformer heads.
// Causal and ring modes take attention sinks: the first n_sink positions stay
// visible next to the window ([KB] §4 "Failure mode 1"; [ST] "What's New"), and
// an optional per-head sink score joins the softmax denominator.  In causal
// mode the band counts the sinks inside a row's window; those before it are
// added after the band, one key at a time in registers.  Symmetric
// mode may take separate global projections ([PP] §5.2): every global key of a
// local row then comes from K_g, V_g (the window tiles drop global positions).
// The global rows themselves (which attend every position, [PP] §4.3) are
// computed from per-block partial states each wave of symmetric mode leaves
// after its own rows (gp_load / gp_finish) and merged by global_combine_kernel.
//
// Tags: [KB] knowledge-base page "Sliding Window Attention" (lizeman.github.io);
// [PP] "Sliding Window Attention: From Local Windows to Global Context"
// (prathamp.com); [ST] "Sliding Window Attention (SWA)" glossary (superteams.ai);
// [G3] "Sliding Window Attention — Gemma 3" study note (ai-engineer-exhaustive.pages.dev).

#include <algorithm>
#include <climits>

#include "swa_internal.h"

namespace swa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct alignas(16) U4 {
  uint32_t w[4];
};

__device__ inline bf16x8 as_bf16x8(U4 u) { return __builtin_bit_cast(bf16x8, u); }

__device__ inline uint32_t pack_bf16(float a, float b) {
  // v_cvt_pk_bf16_f32: round-to-nearest-even on both halves
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

// Minimum and maximum of lo, hi over each half-wave (WHOLE: over the wave)
// with cross-lane VALU moves: DPP inside rows of 16 lanes (lane ^ 1, lane ^ 2,
// then the mirrored lane of the 8- and the 16-lane group), then
// v_permlane16_swap (and v_permlane32_swap).  No LDS round trip, unlike a
// general lane shuffle.
template <bool WHOLE>
__device__ inline void lane_minmax(int &lo, int &hi) {
#define SWA_DPP_STEP(ctrl)                                                   \
  lo = min(lo, __builtin_amdgcn_update_dpp(lo, lo, ctrl, 0xF, 0xF, false)); \
  hi = max(hi, __builtin_amdgcn_update_dpp(hi, hi, ctrl, 0xF, 0xF, false));
  SWA_DPP_STEP(0xB1)   // quad_perm [1, 0, 3, 2]
  SWA_DPP_STEP(0x4E)   // quad_perm [2, 3, 0, 1]
  SWA_DPP_STEP(0x141)  // row_half_mirror
  SWA_DPP_STEP(0x140)  // row_mirror
#undef SWA_DPP_STEP
  auto a = __builtin_amdgcn_permlane16_swap((uint32_t)lo, (uint32_t)lo, false, false);
  auto b = __builtin_amdgcn_permlane16_swap((uint32_t)hi, (uint32_t)hi, false, false);
  lo = min((int)a[0], (int)a[1]);
  hi = max((int)b[0], (int)b[1]);
  if constexpr (WHOLE) {
    auto c = __builtin_amdgcn_permlane32_swap((uint32_t)lo, (uint32_t)lo, false, false);
    auto d = __builtin_amdgcn_permlane32_swap((uint32_t)hi, (uint32_t)hi, false, false);
    lo = min((int)c[0], (int)c[1]);
    hi = max((int)d[0], (int)d[1]);
  }
}

// ---- LDS layouts ---------------------------------------------------------------
#define AS1 __attribute__((address_space(1)))
#define AS3 __attribute__((address_space(3)))
typedef short i16x4 __attribute__((ext_vector_type(4)));

template <int D>
struct Geo {
  static constexpr int ROWB = 2 * D;           // bytes per K/V row
  static constexpr int CPR = D / 8;            // 16-byte chunks per row
  static constexpr int RPI = 1024 / ROWB;      // rows per DMA wave-instruction (4 or 8)
  static constexpr int BN = key_tile(D);       // keys per tile
  static constexpr int NI = BN / RPI;          // DMA instructions per tile and tensor
  static constexpr int TILE_B = BN * ROWB;     // bytes per K (or V) tile
};

// Physical chunk = logical chunk ^ swz(row).
// K: the 16 lanes serviced together read 16 consecutive rows at one logical
//    chunk; swz_k gives them 16 distinct 16-byte bank groups.
// V: a transposing read touches 4 consecutive rows x 4 chunks per half-wave;
//    swz_v spreads those 16 chunks over all bank groups.
template <int D>
__device__ inline int swz_k(int row) { return D == 128 ? (row & 15) : ((row >> 1) & 7); }
template <int D>
__device__ inline int swz_v(int row) { return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1); }


// Workgroup barrier for LDS reuse: waits for this wave's LDS operations but,
// unlike __syncthreads and its fences, not for its global loads and stores.
__device__ inline void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ inline uint32_t lds_addr(const char *p) { return (uint32_t)(uintptr_t)(AS3 const char *)p; }

// Values the compiler cannot prove wave-uniform (they derive from blockIdx and
// the wave index) are pinned to scalar registers.
__device__ inline int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ inline uint32_t uni_u32(uint32_t x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ inline const char *uni_ptr(const char *p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const char *)(((uint64_t)hi << 32) | lo);
}

// HBM -> LDS copies with global_load_lds_dwordx4: lane i's 16 bytes land at
// LDS byte m0 + 16*i.  One call issues a wave's N copies of a tile (1 KB each,
// consecutive in LDS), global address = scalar base + per-lane 32-bit offset.
// Issued from inline assembly so the compiler does not track them: it would
// otherwise wait for every outstanding copy before any LDS read, even of the
// other stage.  The kernel waits (s_waitcnt vmcnt(0)) and barriers before a
// freshly loaded stage is read.  m0 (a reserved register) is restored.
template <int N>
__device__ inline void dma_tile(const char *gbase, const uint32_t *off, uint32_t lds) {
  uint32_t saved;
  if constexpr (N == 4) {
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "global_load_lds_dwordx4 %3, %2\n\t"
        "s_add_u32 m0, m0, 0x400\n\t"
        "global_load_lds_dwordx4 %4, %2\n\t"
        "s_add_u32 m0, m0, 0x400\n\t"
        "global_load_lds_dwordx4 %5, %2\n\t"
        "s_add_u32 m0, m0, 0x400\n\t"
        "global_load_lds_dwordx4 %6, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(uni_u32(lds)), "s"(uni_ptr(gbase)), "v"(off[0]), "v"(off[1]), "v"(off[2]), "v"(off[3])
        : "scc");
  } else if constexpr (N == 1) {
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "global_load_lds_dwordx4 %3, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(uni_u32(lds)), "s"(uni_ptr(gbase)), "v"(off[0]));
  } else {
    static_assert(N == 2, "1, 2 or 4 copies per wave and tile");
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "global_load_lds_dwordx4 %3, %2\n\t"
        "s_add_u32 m0, m0, 0x400\n\t"
        "global_load_lds_dwordx4 %4, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(uni_u32(lds)), "s"(uni_ptr(gbase)), "v"(off[0]), "v"(off[1])
        : "scc");
  }
}

// A whole K/V tile stage from one wave: two copies from the K rows and two
// from the V rows (scalar bases kb, vb, per-lane offsets off[0..3]), landing at
// LDS lds, lds + step, lds + 2 step, lds + 3 step (step = the waves' stride
// through the stage, 1 KB per wave).  One block, no branches.
template <int STEP>
__device__ inline void dma_kv4(const char *kb, const char *vb, const uint32_t *off, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %4, %2\n\t"
      "s_add_u32 m0, m0, %8\n\t"
      "global_load_lds_dwordx4 %5, %2\n\t"
      "s_add_u32 m0, m0, %8\n\t"
      "global_load_lds_dwordx4 %6, %3\n\t"
      "s_add_u32 m0, m0, %8\n\t"
      "global_load_lds_dwordx4 %7, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(uni_u32(lds)), "s"(uni_ptr(kb)), "s"(uni_ptr(vb)), "v"(off[0]), "v"(off[1]), "v"(off[2]),
        "v"(off[3]), "i"(STEP)
      : "scc");
}

// One 4-byte copy per lane (global_load_lds_dword): lane i's word lands at LDS
// byte m0 + 4*i.
__device__ inline void dma_dword(const char *gbase, uint32_t off, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dword %3, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(uni_u32(lds)), "s"(uni_ptr(gbase)), "v"(off));
}

// One 16-byte copy per lane from a full 64-bit address (no scalar base):
// lane i's bytes land at LDS byte m0 + 16*i.
__device__ inline void dma_addr(const void *src, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(uni_u32(lds)), "v"(src));
}

// Wait until at most n of this wave's vector-memory operations are still in
// flight (they complete in issue order), i.e. every copy except the n most
// recent has landed in LDS.  Inline assembly: the compiler does not know about
// the copies and would drop a wait it considers redundant.  n is wave-uniform.
__device__ inline void wait_dma_keep(int n) {
  switch (n) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(1)" ::: "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); break;
    case 3: asm volatile("s_waitcnt vmcnt(3)" ::: "memory"); break;
    case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
    case 5: asm volatile("s_waitcnt vmcnt(5)" ::: "memory"); break;
    case 6: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
    case 7: asm volatile("s_waitcnt vmcnt(7)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
  }
}

__device__ inline bf16x8 tr_read8(const char *p0, const char *p1) {
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((AS3 i16x4 *)p0);
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((AS3 i16x4 *)p1);
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 c = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, c);
}

// Global rows, partial over one wave's 32 keys.  A global row attends every
// position ([PP] §4.3).  The keys at the class positions of a wave's own rows
// (rho + dil*(row0 .. row0+31)) form one block of a partition of [0, T) over
// all waves of the head; the wave scores every global row against that block
// and stores its softmax state (m, l and the unnormalised output), which
// launch_global_combine merges.  The global query, key and value rows come
// from qg, kg, vg when given.
//
// gp_load issues the loads after the banded loop and the out-of-band keys,
// before the epilogue (K in the operand layout, the block's V rows, and for
// d_h = 64 the first 16 global queries), so that they arrive while the
// epilogue runs; gp_finish stages V through the
// wave's output slice (drained by the wave's output stores; LDS operations of
// one wave run in order) for the transposing reads and does the rest.  Rows
// past the class end read the last row instead (those keys are masked, so
// their P is 0 and their finite V adds nothing), and global columns past G
// read position 0 (their results are not stored): every load is in bounds and
// unconditional.
template <int D>
struct GlobalPart {
  // v_mfma_f32_16x16x32_bf16 tiles: 16 global rows per pass, two 16-key halves
  static constexpr int KS = D / 32;  // k-steps of S (32 d per step)
  static constexpr int NV = D / 16;  // 16-byte chunks of the 32 V rows per lane
  static constexpr bool EARLY_Q = D == 64;  // registers allow the queries too
  bf16x8 kf[2][KS];  // K rows (A operand): [key half][k-step]
  u32x4 vr[NV];
  bf16x8 qf[KS];     // global queries (B operand)
};

// 16x16x32 operand layouts: lane l holds A[l % 16][8 (l / 16) + e] and
// B[8 (l / 16) + e][l % 16] (e < 8); the result D[4 (l / 16) + i][l % 16] (i < 4).
template <int D, bool GPROJ>
__device__ inline void gp_load_q(bf16x8 *qf, const FwdArgs &a, int b, int h, int pos) {
  const uint16_t *qsrc = static_cast<const uint16_t *>(GPROJ ? a.qg : a.q);
  const uint16_t *qr = qsrc + (long long)b * a.q_sb + (long long)pos * a.q_st + (long long)h * D;
  const int q4 = (thread_x() & 63) >> 4;
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) qf[ks] = as_bf16x8(*reinterpret_cast<const U4 *>(qr + ks * 32 + q4 * 8));
}

template <int D, bool GPROJ>
__device__ inline void gp_load(GlobalPart<D> &g, const FwdArgs &a, const GlobalList &gl, int b, int h,
                               int kvh, int rho, int dil, int n_cls, int row0) {
  const int lane = thread_x() & 63, l16 = lane & 15, q4 = lane >> 4;
  // the first global positions before the K, V loads, so that the query
  // loads wait for this load only
  const int pos0 = l16 < a.G ? gl.idx[b * a.G + l16] : 0;
  const uint16_t *ksrc = static_cast<const uint16_t *>(GPROJ ? a.kg : a.k);
  const uint16_t *vsrc = static_cast<const uint16_t *>(GPROJ ? a.vg : a.v);
  const long long kv_off = (long long)b * a.k_sb + (long long)kvh * a.k_sh;
  const int last = n_cls - 1;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const uint16_t *kr = ksrc + kv_off + (rho + (long long)dil * min(row0 + mb * 16 + l16, last)) * a.k_st;
#pragma unroll
    for (int ks = 0; ks < GlobalPart<D>::KS; ++ks)
      g.kf[mb][ks] = as_bf16x8(*reinterpret_cast<const U4 *>(kr + ks * 32 + q4 * 8));
  }
  constexpr int CPR = D / 8;
#pragma unroll
  for (int i = 0; i < GlobalPart<D>::NV; ++i) {
    const int idx = i * 64 + lane, r = idx / CPR, ch = idx % CPR;
    g.vr[i] = *reinterpret_cast<const u32x4 *>(vsrc + kv_off + (rho + (long long)dil * min(row0 + r, last)) * a.k_st + ch * 8);
  }
  if constexpr (GlobalPart<D>::EARLY_Q) gp_load_q<D, GPROJ>(g.qf, a, b, h, pos0);
}

// Sum / max of x over the four lanes l % 16 + 16 j (v_permlane16_swap, then
// v_permlane32_swap).
__device__ inline float quad16_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return xhalf_max(fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}
__device__ inline float quad16_add(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return xhalf_add(__uint_as_float(r[0]) + __uint_as_float(r[1]));
}

template <int D, bool GPROJ>
__device__ inline void gp_finish(GlobalPart<D> &g, const FwdArgs &a, const GlobalList &gl, char *vsl,
                                 int b, int h, int rho, int dil, int n_cls, int row0) {
  using Gm = Geo<D>;
  constexpr int DB = D / 16, CPR = D / 8;
  const int lane = thread_x() & 63, l16 = lane & 15, q4 = lane >> 4;
#pragma unroll
  for (int i = 0; i < GlobalPart<D>::NV; ++i) {
    const int idx = i * 64 + lane, r = idx / CPR, ch = idx % CPR;
    *reinterpret_cast<u32x4 *>(vsl + r * Gm::ROWB + ((ch ^ swz_v<D>(r)) * 16)) = g.vr[i];
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
  // V^T operand: lane l takes d = 16 db + l % 16 at keys 4q .. 4q+3 (transposing
  // read of a 4-row x 16-column block per 16 lanes) and 16 + 4q .. 16 + 4q+3
  // (second read, 16 rows on), the key order of its P below
  uint32_t vop[DB];
  {
    const int row = 4 * q4 + (l16 >> 2);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int c = 2 * db + ((l16 >> 1) & 1);
      vop[db] = row * Gm::ROWB + ((c ^ swz_v<D>(row)) * 16) + 8 * (l16 & 1);
    }
  }
  const int last = n_cls - 1;
  const int blk = class_tile_base(a.T, dil, kRowsPerWave, rho) + row0 / kRowsPerWave;
  for (int u0 = 0; u0 < a.G; u0 += 16) {
    const int u = u0 + l16;
    if (!GlobalPart<D>::EARLY_Q || u0 > 0) gp_load_q<D, GPROJ>(g.qf, a, b, h, u < a.G ? gl.idx[b * a.G + u] : 0);
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    f32x4 sg[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      sg[mb] = f32x4{};
#pragma unroll
      for (int ks = 0; ks < GlobalPart<D>::KS; ++ks)
        sg[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(g.kf[mb][ks], g.qf[ks], sg[mb], 0, 0, 0);
    }
    // element (mb, i) holds key row0 + 16 mb + 4q + i for global row u
    float mx = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (row0 + 16 * mb + 4 * q4 + i > last) sg[mb][i] = -INFINITY;
        mx = fmaxf(mx, sg[mb][i]);
      }
    const float mg = quad16_max(mx) * a.sl2;  // finite: key row0 exists
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) sg[mb][i] = __builtin_amdgcn_exp2f(fmaf(sg[mb][i], a.sl2, -mg));
    U4 pw;
    pw.w[0] = pack_bf16(sg[0][0], sg[0][1]);
    pw.w[1] = pack_bf16(sg[0][2], sg[0][3]);
    pw.w[2] = pack_bf16(sg[1][0], sg[1][1]);
    pw.w[3] = pack_bf16(sg[1][2], sg[1][3]);
    // row sum over the rounded weights the product uses (v_dot2 against ones)
    const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
    float rs = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw.w[w]), ones, rs, false);
    const float lg = quad16_add(rs);
    // every lane takes part in the reads and products (each output column
    // needs the operand rows of all lanes); only global rows that exist store
    float *dst = a.gws + ((((long long)b * a.Hq + h) * a.G + min(u, a.G - 1)) * a.gnb + blk) * (D + 4);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const char *p0 = vsl + vop[db];
      const f32x4 og = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tr_read8(p0, p0 + 16 * Gm::ROWB),
                                                               as_bf16x8(pw), f32x4{}, 0, 0, 0);
      if (u < a.G)
        *reinterpret_cast<float4 *>(dst + db * 16 + 4 * q4) = make_float4(og[0], og[1], og[2], og[3]);
    }
    if (u < a.G && q4 == 0) *reinterpret_cast<float2 *>(dst + D) = make_float2(mg, lg);
  }
}

// ---- the kernel ------------------------------------------------------------------

template <int N>
struct IntC {
  static constexpr int value = N;
};

// Copy stages of the symmetric (Longformer) kernel.
#ifndef SWA_SYM_STAGES
#define SWA_SYM_STAGES 2
#endif

// Largest growth (log2 units) of a row max tolerated before the running
// reference max is raised and O, l are rescaled.
constexpr float kLazy = 8.f;

// NW waves per workgroup; three waves per SIMD (12 per CU) bound the registers.
// MODE: kCausal, kSymmetric, kRing, kCausalSink, kSymmetricProj or kCausalDil
// (FwdMode).
template <int D, int MODE, int NW>
__global__ __launch_bounds__(64 * NW, (D == 64 && MODE == kSymmetric) ? 16 / NW
                                      : (12 / NW) > 0 ? 12 / NW : 1) void fwd_kernel(
    const FwdArgs a, const GlobalList gl) {
  constexpr bool GPROJ = MODE == kSymmetricProj;  // separate global projections
  constexpr bool SYM = MODE == kSymmetric || GPROJ;
  constexpr bool RING = MODE == kRing;
  constexpr bool CSINK = MODE == kCausalSink;  // causal with sink tokens / scores
  constexpr bool CDIL = MODE == kCausalDil;    // causal, dilated heads (residue classes)
  constexpr bool SCORE = CSINK || RING;        // may carry per-head sink scores
  using Gm = Geo<D>;
  // NST stages, each a row-major K tile followed by a V tile (swizzled
  // chunks); copies run NST-1 tiles ahead of the compute.  After the loop the
  // same memory stages the output rows.
  constexpr int STAGE_B = 2 * Gm::TILE_B;
  constexpr int NST = SYM ? SWA_SYM_STAGES : 2;
  // ring mode: the slot positions of stage st sit at byte 256 st, ahead of
  // the stages, so every read of them is one base register plus an immediate
  constexpr int SPA = RING ? 1024 : 0;
  static_assert(!RING || NST * 256 <= SPA, "slot positions fit ahead of the stages");
  constexpr int OST_B = NW * kRowsPerWave * D * 2;
  constexpr int SMEM_B = (SPA + NST * STAGE_B > OST_B) ? SPA + NST * STAGE_B : OST_B;
  // symmetric mode: K rows then V rows of the (at most kValuGlobals) global
  // keys, staged once for the after-the-band pass
  // (causal sink mode: the K rows then V rows of the sink tokens, likewise)
  constexpr int GKV_ROWS = MODE == kSymmetric ? kValuGlobals : MODE == kCausalSink ? kMaxSinks : 0;
  constexpr int GKV_B = 2 * GKV_ROWS * Gm::ROWB;
  __shared__ __attribute__((aligned(1024))) char smem[SMEM_B + GKV_B];
  constexpr int KS_QK = D / 16;  // k-steps of S = Q K^T
  constexpr int DB = D / 32;     // 32-wide d blocks of O^T
  constexpr int BN = Gm::BN;     // keys per tile
  constexpr int KB = BN / 32;    // 32-key blocks of S^T per tile

  const int tid = thread_x();
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  __builtin_assume(wave >= 0 && wave < NW);
  const int lq = lane & 31, lh = lane >> 5;

  // -------- work decode
  int b, h, kvh, row0;  // row0: first query row (class index in symmetric mode)
  int rho = 0, dil = 1, n_cls;  // residue class, dilation, class length
  int tile_row0, tile_rows;     // workgroup's query rows (for the tile schedule)
  if constexpr (!SYM && !CDIL) {
    const int nblk = a.B * a.n_hg * a.n_qt;
    const int lid = xcd_remap(group_x(), nblk);
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
    // (batch, head or head group, residue class, query tile); in a dilated
    // causal head group the waves take P heads x NW/P row blocks as above
    const int nblk = a.B * a.tiles_per_batch;
    // Dilated causal heads differ in work (shorter classes put more rows in
    // the ramp), so the host cuts the enumeration into 8 ranges of equal work,
    // one per XCD: each XCD runs consecutive tiles of few classes, whose bands
    // share its L2.  Workgroups past their XCD's range exit at once.
    int lid;
    if constexpr (CDIL) {
      const int x = group_x() & 7, i = group_x() >> 3;
      lid = a.xcd_off[x] + i;
      if (lid >= a.xcd_off[x + 1]) return;
    } else {
      lid = xcd_remap(group_x(), nblk);
    }
    b = lid / a.tiles_per_batch;
    const int rem = lid % a.tiles_per_batch;
    // find the head (group): head_off[g] <= rem < head_off[g+1]
    int lo = 0, hi = (SYM ? a.Hq : a.n_hg) - 1;
    while (lo < hi) {
      const int mid = uni((lo + hi + 1) >> 1);
      if (a.head_off[mid] <= rem) lo = mid; else hi = mid - 1;
    }
    lo = uni(lo);
    {
      // the 16-bit entry from its 32-bit word, so the load is a scalar one
      const uint32_t w = reinterpret_cast<const uint32_t *>(a.dil)[lo >> 1];
      dil = (lo & 1) ? (int)(w >> 16) : (int)(w & 0xffffu);
    }
    int tile;
    class_tile_decode(a.T, dil, a.BM, rem - a.head_off[lo], &rho, &tile);
    n_cls = class_len(class_split(a.T, dil), rho);
    if constexpr (CDIL) tile = ceil_div(n_cls, a.BM) - 1 - tile;  // heavy (full-band) tiles first
    tile_row0 = tile * a.BM;
    if constexpr (SYM) {
      h = lo;
      kvh = h;
      row0 = tile_row0 + wave * kRowsPerWave;
    } else {
      h = lo * a.P + (wave % a.P);
      kvh = h / a.group;
      row0 = tile_row0 + (wave / a.P) * kRowsPerWave;
    }
  }
  b = uni(b);
  h = uni(h);
  kvh = uni(kvh);
  rho = uni(rho);
  dil = uni(dil);
  n_cls = uni(n_cls);
  tile_row0 = uni(tile_row0);
  row0 = uni(row0);
  const int t1_valid = min(tile_row0 + a.BM, n_cls) - 1;  // last valid row of the tile

  const uint16_t *qg = static_cast<const uint16_t *>(a.q);
  const uint16_t *kg = static_cast<const uint16_t *>(a.k);
  const uint16_t *vg = static_cast<const uint16_t *>(a.v);
  // position of class row i: rho + dil*i (dil = 1, rho = 0 in causal mode)
  const long long q_rowstride = a.q_st * dil;
  const long long k_rowstride = a.k_st * dil;
  const long long k_rho = (long long)rho * a.k_st;
  const uint16_t *kbase = kg + (long long)b * a.k_sb + (long long)kvh * a.k_sh;
  const uint16_t *vbase = vg + (long long)b * a.k_sb + (long long)kvh * a.k_sh;
  const int n_keyrows = RING ? a.S : n_cls;  // key rows of this (batch, head)

  // ring mode: this lane's query position, loaded ahead of Q so that waiting
  // for it does not wait for Q
  int q_pos_ld = 0;
  if constexpr (RING)
    if (row0 + lq < n_cls) q_pos_ld = a.q_pos[(long long)b * a.T + row0 + lq];

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

  // -------- global keys of symmetric mode, sink tokens of causal sink mode ->
  // LDS: the K rows, then (GKV_ROWS rows further) the V rows, copied straight
  // into LDS, RPI rows per wave instruction.  They are issued after Q (they
  // wait for the global positions' scalar loads) and before the tile copies,
  // so the first tile step's wait covers them and its barrier publishes them
  // to the other waves; they are read after the band.  Rows past the last one
  // repeat it (inside the GKV_ROWS-row regions).
  char *const gkv = smem + SMEM_B;
  // sink tokens that exist (positions below both n_sink and T)
  const int n_sink = CSINK ? min(a.n_sink, n_cls) : 0;
  if constexpr (MODE == kSymmetric || CSINK) {
    constexpr int RPI = Gm::RPI, CPR = D / 8;
    const int n_rows = CSINK ? n_sink : a.G;
    const int n_i = (n_rows + RPI - 1) / RPI;  // copies per tensor
    const int sub = lane / CPR;                 // this lane's row in a copy
    for (int i = wave; i < 2 * n_i; i += NW) {
      const int isv = i >= n_i;
      const int r0i = (isv ? i - n_i : i) * RPI;
      int pos = min(r0i + sub, n_rows - 1);  // sinks: positions 0 .. n_sink-1
      if constexpr (MODE == kSymmetric) {
        // the global positions, read with wave-uniform indices
#pragma unroll
        for (int k = 0; k < RPI; ++k) {
          const int pk = gl.idx[b * a.G + min(r0i + k, n_rows - 1)];
          pos = sub == k ? pk : pos;
        }
      }
      const uint16_t *src = (isv ? vbase : kbase) + (long long)pos * a.k_st + (lane % CPR) * 8;
      dma_addr(src, lds_addr(gkv) + (uint32_t)((isv * GKV_ROWS + r0i) * Gm::ROWB));
    }
  }

  // -------- schedule
  TileRange tr;
  if constexpr (RING) tr = {0, ceil_div(a.S, BN) - 1};  // every slot tile
  else if constexpr (!SYM) tr = causal_tile_range(tile_row0, t1_valid, a.W, BN);
  else tr = sym_tile_range(tile_row0, t1_valid, a.W, n_cls, BN);
  tr.lo = uni(tr.lo);
  tr.hi = uni(tr.hi);
  const int n_win = tr.hi - tr.lo + 1;
  // extra tiles after the window: the global keys when they have projections
  // of their own (sink tokens and shared-projection globals are staged apart)
  const int n_glob = GPROJ ? ceil_div(a.G, BN) : 0;
  const int n_tiles = n_win + n_glob;
  // this wave's valid rows [row0, w_last] and the window tiles they need
  const int w_last = min(row0 + kRowsPerWave, n_cls) - 1;
  TileRange wr{1, 0};
  if (w_last >= row0) {
    if constexpr (RING) wr = tr;
    else if constexpr (!SYM) wr = causal_tile_range(row0, w_last, a.W, BN);
    else wr = sym_tile_range(row0, w_last, a.W, n_cls, BN);
  }
  wr.lo = uni(wr.lo);
  wr.hi = uni(wr.hi);
  const bool has_rows = w_last >= row0;
  // Per tile, one unsigned compare each: window tile j is computed iff
  // j - jc_lo <= jc_span, and needs no mask iff j - jf_lo <= jf_span (the
  // full tiles of the wave's rows, a sub-range of its window tiles).
  int jc_lo = 1 << 30, jf_lo = 1 << 30;
  unsigned jc_span = 0, jf_span = 0;
  if (has_rows) {
    jc_lo = wr.lo - tr.lo;
    jc_span = (unsigned)(wr.hi - wr.lo);
    if constexpr (!RING) {
      TileRange fr;
      if constexpr (!SYM) fr = causal_full_range(row0, w_last, a.W, BN, n_cls);
      else fr = sym_full_range(row0, w_last, a.W, BN, n_cls);
      fr.lo = max(fr.lo, wr.lo);
      fr.hi = min(fr.hi, wr.hi);
      if (fr.lo <= fr.hi) {
        jf_lo = fr.lo - tr.lo;
        jf_span = (unsigned)(fr.hi - fr.lo);
      }
    }
  }
  // the 32-key blocks every row of the wave attends in full (64-key tiles)
  TileRange fb{1 << 30, 1 << 30};
  if constexpr (!RING && KB > 1) {
    if (has_rows) {
      const TileRange f = SYM ? sym_full_range(row0, w_last, a.W, 32, n_cls)
                              : causal_full_range(row0, w_last, a.W, 32, n_cls);
      if (f.lo <= f.hi) fb = f;
    }
    fb.lo = uni(fb.lo);
    fb.hi = uni(fb.hi);
  }
  // 64-key tiles: the first window tile of a wave may start, and its last
  // window tile end, with a whole 32-key block that no row of the wave attends
  // (its band starts or ends mid-tile).  That block is neither multiplied nor
  // exponentiated: tile jh0 computes only its block 1, tile jh1 only block 0.
  // (A tile cannot be both jh0 and jh1: both its blocks would then lie outside
  // the band, and the tile would not be in the wave's range.)
  int jh0 = 1 << 30, jh1 = 1 << 30;
  if constexpr (!RING && KB > 1) {
    if (has_rows) {
      // the 32-key blocks some row of the wave attends: [ab.lo, ab.hi]
      const TileRange ab = SYM ? sym_tile_range(row0, w_last, a.W, n_cls, 32)
                               : causal_tile_range(row0, w_last, a.W, 32);
      if (ab.lo & 1) jh0 = wr.lo - tr.lo;     // block 2 wr.lo < ab.lo
      if (!(ab.hi & 1)) jh1 = wr.hi - tr.lo;  // block 2 wr.hi + 1 > ab.hi
    }
    jh0 = uni(jh0);
    jh1 = uni(jh1);
  }
  jc_lo = uni(jc_lo);
  jf_lo = uni(jf_lo);
  jc_span = (unsigned)uni((int)jc_span);
  jf_span = (unsigned)uni((int)jf_span);

  // -------- DMA addressing.  A stage takes 2*NI wave instructions of 1 KB:
  // instruction i < NI copies K rows i*RPI .. i*RPI+RPI-1, instruction NI + i
  // the same V rows, to stage byte 1024*i.  Lane l lands at byte 16*l of its
  // instruction's 1 KB, i.e. row i*RPI + l/CPR, physical chunk l%CPR, so it
  // loads logical chunk (l%CPR) ^ swz(row).  Wave w issues instructions
  // w, w+NW, ...  Rows of a window tile are consecutive class rows, so the
  // per-lane byte offsets are fixed and each tile adds a uniform base.
  constexpr int NSLOT = (2 * Gm::NI + NW - 1) / NW;
  const long long rs_b = k_rowstride * 2;  // bytes between consecutive class rows
  uint32_t loff[NSLOT];
#pragma unroll
  for (int t = 0; t < NSLOT; ++t) {
    const int i = wave + t * NW;
    const int r = (i % Gm::NI) * Gm::RPI + lane / Gm::CPR;
    const int p = lane % Gm::CPR;
    loff[t] = (uint32_t)(r * rs_b) + (p ^ (i >= Gm::NI ? swz_v<D>(r) : swz_k<D>(r))) * 16;
  }
  // Copy sources as byte distances from the K base, so a copy picks its source
  // by adding offsets (each choice between a distance and zero).  A choice
  // between two captured pointer variables would be merged into one load
  // through a selected capture address, which keeps every variable the
  // lambdas capture in scratch memory.
  const char *kb8 = reinterpret_cast<const char *>(kbase);
  const long long d_v = (long long)((uintptr_t)vbase - (uintptr_t)kbase);  // V rows
  // tiles of global keys read K_g, V_g with separate projections
  const long long kv_off = ((long long)b * a.k_sb + (long long)kvh * a.k_sh) * 2;
  const long long d_gk =
      GPROJ ? (long long)((uintptr_t)a.kg + kv_off - (uintptr_t)kbase) : 0;
  const long long d_gvk =  // (V_g - V) - (K_g - K)
      GPROJ ? (long long)(((uintptr_t)a.vg - (uintptr_t)a.v) - ((uintptr_t)a.kg - (uintptr_t)a.k))
            : 0;
  // DMA of the K and V rows of tile j (window tiles j < n_win, then tiles of
  // global keys) into the stage at LDS address `stage`.
  // Four copies per wave, the first two K rows and the last two V rows (four
  // waves): a whole window tile goes out as one branch-free block.
  constexpr bool KV4 = NSLOT == 4 && NSLOT * NW == 2 * Gm::NI && Gm::NI == 2 * NW;
  // window tiles j <= jw_hi hold BN valid key rows
  const int jw_hi = uni(min(n_keyrows / BN - 1, tr.hi) - tr.lo);
  const uint32_t a_s0 = lds_addr(smem) + (uint32_t)SPA;  // the stages
  auto issue = [&](int j, int si) {  // into stage si
    const uint32_t stage = a_s0 + (uint32_t)(si * STAGE_B);
    const int kt = (j < n_win) ? tr.lo + j : 0;  // key tile (0 past the window)
    const bool whole = (j < n_win) ? j <= jw_hi : (!SYM && BN <= n_keyrows);
    const long long base = (k_rho + (long long)kt * BN * k_rowstride) * 2;
    if (KV4 && j <= jw_hi) {
      const char *kt8 = kb8 + base;
      dma_kv4<NW * 1024>(kt8, kt8 + d_v, loff, stage + (uint32_t)wave * 1024u);
    } else {
#pragma unroll
    for (int t = 0; t < NSLOT; ++t) {
      const int i = wave + t * NW;
      if (i < 2 * Gm::NI) {
        const bool isv = i >= Gm::NI;
        long long src = isv ? d_v : 0;
        if (GPROJ && j >= n_win) src += d_gk + (isv ? d_gvk : 0);
        const char *g8 = kb8 + src;
        const uint32_t ld = stage + (uint32_t)i * 1024u;
        if (whole) {
          // whole tile inside the class: uniform base + fixed lane offsets
          dma_tile<1>(g8 + base, &loff[t], ld);
        } else {
          // ragged last tile (rows clamped to the last valid row; the mask
          // removes them) or a tile of global keys (absolute positions)
          const int r = (i % Gm::NI) * Gm::RPI + lane / Gm::CPR;
          const int p = lane % Gm::CPR;
          long long o;
          if (j < n_win || !SYM) {
            const int sr = min(kt * BN + r, n_keyrows - 1);
            o = (k_rho + (long long)sr * k_rowstride) * 2;
          } else {
            const int u = min((j - n_win) * BN + r, a.G - 1);
            o = (long long)gl.idx[b * a.G + u] * a.k_st * 2;
          }
          const uint32_t off = (uint32_t)o + (p ^ (isv ? swz_v<D>(r) : swz_k<D>(r))) * 16;
          dma_tile<1>(g8, &off, ld);
        }
      }
    }
    }
    if constexpr (RING) {
      // the tile's slot positions (lane i: slot tile*BN + i, clamped; the
      // mask ignores slots past S)
      if (wave == NW - 1) {
        const int slot = min((tr.lo + j) * BN + lane, a.S - 1);
        dma_dword(reinterpret_cast<const char *>(a.slot_pos + (long long)b * a.S),
                  (uint32_t)slot * 4u, lds_addr(smem) + (uint32_t)(si * 256));
      }
    }
  };

  // -------- operand read offsets (bytes within a tile)
  // K (A operand of S^T): lane reads row 32kb + lq, logical chunk 2kk + lh.
  uint32_t kop[KS_QK];
#pragma unroll
  for (int kk = 0; kk < KS_QK; ++kk) {
    kop[kk] = lq * Gm::ROWB + (((2 * kk + lh) ^ swz_k<D>(lq)) * 16);
    // kept whole, so each read is one ds_read with the stage as its offset
    asm volatile("" : "+v"(kop[kk]));
  }
  // V^T (A operand of O^T): two transposing reads per 16-key step.  In each
  // group of 16 lanes, source lane s addresses row 16kk + 4hh + s/4 at columns
  // 32db + 16dg + 4(s%4) .. +3, so output lane i of the group receives column
  // 32db + 16dg + i of those 4 rows; the second read adds 8 rows.  The 8 keys
  // a lane gets are 16kk + {4hh..4hh+3, 8+4hh..8+4hh+3}, the order in which
  // the P^T B operand holds them.
  uint32_t vop[DB];
  {
    const int grp = lane >> 4, sl = lane & 15;
    const int hh = grp >> 1, dg = grp & 1;
    const int row = 4 * hh + (sl >> 2);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int c = 4 * db + 2 * dg + ((sl >> 1) & 1);
      vop[db] = row * Gm::ROWB + ((c ^ swz_v<D>(row)) * 16) + 8 * (sl & 1);
      asm volatile("" : "+v"(vop[db]));
    }
  }

  // -------- running softmax state (lane owns query row lq; both half-waves agree)
  f32x16 acc_o[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) acc_o[i] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  // exponent reference (m_run, or 0 while m_run = -inf) and the raw-score
  // threshold above which a row triggers the lazy rescale, (m_run + kLazy) /
  // sl2; both change only when m_run does
  float m_use = 0.f, m_thr = -INFINITY;
  const int my_row = row0 + lq;

  // ---- building blocks.  They work on NB consecutive 32-key blocks of the
  // staged tile starting at block B0 (B0 = 0, NB = KB: the whole tile), both
  // compile-time constants.  Accumulator element (kb, e) of S^T holds key
  // 32(B0 + kb) + 8(e/4) + 4lh + (e%4) of the tile, for query row my_row.
  auto qk = [&](const char *ks, f32x16 *sv, auto b0, auto nb) {
    constexpr int B0 = decltype(b0)::value, NB = decltype(nb)::value;
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) sv[kb] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < KS_QK; ++kk)
#pragma unroll
      for (int kb = 0; kb < NB; ++kb) {
        const U4 u = *reinterpret_cast<const U4 *>(ks + (B0 + kb) * 32 * Gm::ROWB + kop[kk]);
        sv[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(u), qf[kk], sv[kb], 0, 0, 0);
      }
  };
  // this lane's share of its row max over the blocks (its half of the keys),
  // in raw score units: three-input max chains
  auto rowmax = [&](const f32x16 *sv, auto nb) {
    constexpr int NB = decltype(nb)::value;
    float mx = fmaxf(fmaxf(sv[0][0], sv[0][1]), sv[0][2]);
#pragma unroll
    for (int e = 3; e < 15; e += 2) mx = fmaxf(fmaxf(mx, sv[0][e]), sv[0][e + 1]);
    mx = fmaxf(mx, sv[0][15]);
#pragma unroll
    for (int kb = 1; kb < NB; ++kb)
#pragma unroll
      for (int e = 0; e < 16; e += 2) mx = fmaxf(fmaxf(mx, sv[kb][e]), sv[kb][e + 1]);
    return mx;
  };
  // The reference max m_run is only raised when some row of the wave would
  // otherwise see p = 2^(s - m_run) above 2^kLazy; l and O share the same
  // reference, so the result is unchanged and O is rarely rescaled.  mx is a
  // lane's share of its row max in raw score units: a row's max passes the
  // threshold iff one of its two halves does, so the test needs no exchange
  // with the partner half-wave; the rescale takes the whole row's max.
  auto rescale = [&](float mx_half) {
    if (__builtin_amdgcn_ballot_w64(mx_half > m_thr) != 0) {
      const float mx = xhalf_max(mx_half);
      const float m_new = fmaxf(m_run, mx * a.sl2);
      const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < DB; ++i) acc_o[i] *= alpha;
      m_run = m_new;
      m_use = (m_run == -INFINITY) ? 0.f : m_run;
      m_thr = (m_run == -INFINITY) ? -INFINITY : (m_run + kLazy) / a.sl2;
    }
  };
  // P = 2^(s sl2 - m) over the blocks, packed to bf16 as the B operand of the
  // P.V product: 2 NB key steps of 16
  auto exp_pack = [&](f32x16 *sv, U4 *pu, auto nb) {
    constexpr int NB = decltype(nb)::value;
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) sv[kb][e] = __builtin_amdgcn_exp2f(fmaf(sv[kb][e], a.sl2, -m_use));
#pragma unroll
    for (int kk = 0; kk < 2 * NB; ++kk) {
      const int kb = kk >> 1, e0 = (kk & 1) * 8;
#pragma unroll
      for (int w = 0; w < 4; ++w) pu[kk].w[w] = pack_bf16(sv[kb][e0 + 2 * w], sv[kb][e0 + 2 * w + 1]);
    }
    // Row sum of the P the product uses (bf16 pairs, v_dot2 against ones,
    // fp32 accumulation): this lane's keys only; the half-wave partner's
    // share is added once, before the epilogue.
    const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
#pragma unroll
    for (int kk = 0; kk < 2 * NB; ++kk)
#pragma unroll
      for (int w = 0; w < 4; ++w)
        l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pu[kk].w[w]), ones, l_run, false);
  };
  // O^T += V^T P^T : key steps of 16 over the blocks
  auto pv = [&](const char *vs, const U4 *pu, auto b0, auto nb) {
    constexpr int B0 = decltype(b0)::value, NB = decltype(nb)::value;
#pragma unroll
    for (int kk = 0; kk < 2 * NB; ++kk) {
      const bf16x8 pb = as_bf16x8(pu[kk]);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const char *p0 = vs + (2 * B0 + kk) * 16 * Gm::ROWB + vop[db];
        const bf16x8 vt = tr_read8(p0, p0 + 8 * Gm::ROWB);
        acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vt, pb, acc_o[db], 0, 0, 0);
      }
    }
  };
  // With separate global projections (or many globals): columns of window
  // tile j holding a global position of this residue class (uniform; the loop
  // runs over the globals).  The window tiles mask them and the tile of global
  // keys attends every global, so a global inside a row's window is counted
  // once (and, with separate projections, read through K_g).  Plain symmetric
  // mode adds its few global keys after the band instead (see below).
  auto glob_cols = [&](int j) -> uint64_t {
    uint64_t m = 0;
    if constexpr (GPROJ) {
      if (j < n_win && a.G > 0) {
        const int c0 = (tr.lo + j) * BN;
        for (int u = 0; u < a.G; ++u) {
          const int d = gl.idx[b * a.G + u] - rho;
          if (d >= 0 && d % dil == 0) {
            const int c = d / dil - c0;
            if (c >= 0 && c < BN) m |= 1ull << c;
          }
        }
      }
    }
    return m;
  };
  // every (valid row of this wave, key) pair of window tile j attended?
  // (tiles of global keys, j >= n_win, lie outside the range: always masked)
  auto tile_full = [&](int j) { return (unsigned)(j - jf_lo) <= jf_span; };
  // Ring mode: this lane's query position and the wave's position range.
  int my_pos = 0, pos_lo = 0, pos_hi = 0;
  if constexpr (RING) {
    const bool ok = my_row < n_cls;
    my_pos = q_pos_ld;
    int lo = ok ? my_pos : INT_MAX, hi = ok ? my_pos : INT_MIN;
    lane_minmax<false>(lo, hi);  // both half-waves hold the same 32 rows
    pos_lo = uni(lo);
    pos_hi = uni(hi);
    asm volatile("" ::"v"(my_pos));
  }
  // Ring tile class for the rows of this wave (query positions in
  // [pos_lo, pos_hi]): 1 = every (row, slot) pair attended (all slots exist,
  // are filled and lie in the window of every row), 0 = no slot lies in the
  // window of any row (nor is a sink), so the tile adds nothing and is
  // skipped, 2 = partial (masked).
  auto slot_pos_of = [&](int st) {  // slot positions of the tile in stage st
    return reinterpret_cast<const int *>(smem + st * 256);
  };
  // lanes whose slot (lane % BN) of tile j exists, from the uniform count
  auto slot_lanes = [&](int j) -> uint64_t {
    const int n_in = min(BN, a.S - (tr.lo + j) * BN);
    if constexpr (BN == 64) return n_in >= 64 ? ~0ull : (1ull << n_in) - 1;
    const uint64_t m = n_in >= 32 ? 0xffffffffull : (1ull << n_in) - 1;
    return m | (m << 32);
  };
  auto ring_class = [&](int st, int j) {
    const int n_in = min(BN, a.S - (tr.lo + j) * BN);
    const int sp = slot_pos_of(st)[lane % BN];
    const bool live = sp >= 0 && sp <= pos_hi &&
                      ((long long)sp > (long long)pos_lo - a.W || sp < a.n_sink);
    if ((__builtin_amdgcn_ballot_w64(live) & slot_lanes(j)) == 0) return 0;
    // every slot in the window of every row (with 32 slots both half-waves
    // hold them all)
    const bool all_in = sp >= 0 && (long long)sp > (long long)pos_hi - a.W && sp <= pos_lo;
    const bool full = n_in == BN && __builtin_amdgcn_ballot_w64(all_in) == ~0ull;
    return full ? 1 : 2;
  };
  // Ring mask: slot k of the tile (k < S) is attended iff its position p has
  // p >= 0 and my_pos - W < p <= my_pos.
  auto ring_mask = [&](int st, int j, f32x16 *sv) {
    // slot c + 4 lh (c the element's constant part) exists iff c < lim
    const int lim = min(BN, a.S - (tr.lo + j) * BN) - 4 * lh;
    const int *spl = slot_pos_of(st) + 4 * lh;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int c0 = kb * 32 + 8 * g4;
        const int4 p4 = *reinterpret_cast<const int4 *>(spl + c0);
        const int pv[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int p = pv[i];
          const bool ok = c0 + i < lim && p >= 0 && p <= my_pos &&
                          (p > my_pos - a.W || p < a.n_sink);
          if (!ok) sv[kb][4 * g4 + i] = -INFINITY;
        }
      }
  };
  // Ring mode: value rows of the slots of a staged tile that hold no token
  // (negative position, or past the ring's end) are zeroed in LDS before any
  // wave reads the tile.  Their weights are 0 already, but 0 times the NaN or
  // Inf bits an unwritten slot may hold would not be.  Every wave sees the
  // same slot positions, so all take the same branch and the same barrier.
  auto ring_zero_holes = [&](int st, int j) {
    const int sp = slot_pos_of(st)[lane % BN];
    const uint64_t hole = __builtin_amdgcn_ballot_w64(sp < 0) | ~slot_lanes(j);
    if (hole == 0) return;
    constexpr int CPR = D / 8, RPW = 64 / CPR;  // 16-byte chunks per row, rows per store
    char *vt = smem + SPA + st * STAGE_B + Gm::TILE_B;
#pragma unroll
    for (int r0 = wave * RPW; r0 < BN; r0 += NW * RPW) {
      const int row = r0 + lane / CPR;
      if ((hole >> row) & 1ull)
        *reinterpret_cast<u32x4 *>(vt + row * Gm::ROWB + (lane % CPR) * 16) = u32x4{0, 0, 0, 0};
    }
    lds_barrier();
  };
  // Attended keys of row my_row inside the window, [lo_key, hi_key]: the
  // causal predicate (t-W < s <= t) or the symmetric one (|i-j| <= r), cut at
  // the class length.
  int lo_key, hi_key;
  row_key_bounds(SYM, my_row, a.W, n_cls, &lo_key, &hi_key);
  // mask of a partial tile over the blocks B0 .. B0+NB-1: the window
  // predicate (global positions left out when gcols marks some), or for a
  // tile of global keys the existing globals
  auto mask = [&](int j, f32x16 *sv, uint64_t gcols, auto b0, auto nb) {
    constexpr int B0 = decltype(b0)::value, NB = decltype(nb)::value;
    if (j < n_win) {
      // key of element (kb, e) = tile base + 4*lh + c(kb, e); compare c with
      // this lane's bounds shifted to the same origin
      const int base = (tr.lo + j) * BN + 4 * lh;
      const int lo = lo_key - base, hi = hi_key - base;
      if (GPROJ && gcols) {
        // global positions of this class in the tile: counted in the global tile
        const uint64_t gl_lane = gcols >> (4 * lh);
#pragma unroll
        for (int kb = 0; kb < NB; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int c = (B0 + kb) * 32 + 8 * (e >> 2) + (e & 3);
            if (c < lo || c > hi || ((gl_lane >> c) & 1)) sv[kb][e] = -INFINITY;
          }
        return;
      }
      // one unsigned compare per element: c in [lo, hi] iff c - lo <= hi - lo
      // (an empty range moves lo out of reach)
      const int lo2 = hi >= lo ? lo : (1 << 30);
      const uint32_t span = hi >= lo ? (uint32_t)(hi - lo) : 0u;
#pragma unroll
      for (int kb = 0; kb < NB; ++kb) {
        if constexpr (KB > 1) {
          // a 32-key block inside every row's window needs no mask
          const int blk = (tr.lo + j) * (BN / 32) + B0 + kb;
          if ((unsigned)(blk - fb.lo) <= (unsigned)(fb.hi - fb.lo)) continue;
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int c = (B0 + kb) * 32 + 8 * (e >> 2) + (e & 3);
          if ((uint32_t)(c - lo2) > span) sv[kb][e] = -INFINITY;
        }
      }
      return;
    }
    if constexpr (!SYM) return;
    // Tile of global keys: column c holds global u0 + c.  Every existing global
    // is attended here; the window tiles leave global positions out
    // (glob_cols), so each key is counted once.
    const int hi = min(a.G - (j - n_win) * BN, BN) - 1 - 4 * lh;  // this lane's origin
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int c = (B0 + kb) * 32 + 8 * (e >> 2) + (e & 3);
        if (c > hi) sv[kb][e] = -INFINITY;
      }
  };

  // ---- main loop: tile j is computed from stage j % NST while the copies of
  // tiles j+1 .. j+NST-1 are in flight.  Step j waits for its own tile and
  // barriers (so every wave is also done with tile j-1), then reuses tile
  // j-1's stage for tile j+NST-1.  Unrolled by the NST stages so every LDS
  // operand address is a fixed register plus an immediate offset.
  constexpr int NCOPY = NSLOT;  // copies per wave and tile
  static_assert((2 * Gm::NI) % NW == 0, "every wave issues the same number of copies");
  auto step = [&](int j, auto stage) {
    constexpr int st = decltype(stage)::value;
    wait_dma_keep(NST == 2 ? 0 : min(n_tiles - 1 - j, NST - 2) * NCOPY);
    __syncthreads();
    if (j + NST - 1 < n_tiles) issue(j + NST - 1, (st + NST - 1) % NST);
    // a wave computes the tiles of its rows' band and the tiles of global keys
    char *ks = smem + SPA + st * STAGE_B;
    int rc = 1;  // ring mode: tile class (0 = nothing attended, skip)
    if constexpr (RING) {
      ring_zero_holes(st, j);
      rc = has_rows ? ring_class(st, j) : 0;
    }
    const bool comp = (n_glob > 0 && j >= n_win) ? has_rows : (unsigned)(j - jc_lo) <= jc_span;
    // the computed blocks B0 .. B0+NB-1 of the tile
    auto blocks = [&](auto b0, auto nb) {
      constexpr int NB = decltype(nb)::value;
      f32x16 sv[NB];
      U4 pu[2 * NB];
      qk(ks, sv, b0, nb);
      if constexpr (RING) {
        if (rc == 2) ring_mask(st, j, sv);
      } else {
        const uint64_t gcols = glob_cols(j);
        if (gcols || !tile_full(j)) mask(j, sv, gcols, b0, nb);
      }
      rescale(rowmax(sv, nb));
      exp_pack(sv, pu, nb);
      pv(ks + Gm::TILE_B, pu, b0, nb);
    };
    if (rc != 0 && comp) {
      if constexpr (!RING && KB > 1) {
        // the two 32-key halves in turn, each with its own max test; a half
        // that no row of the wave attends is skipped
        if (j != jh0) blocks(IntC<0>{}, IntC<1>{});
        if (j != jh1) blocks(IntC<1>{}, IntC<1>{});
      } else {
        blocks(IntC<0>{}, IntC<KB>{});
      }
    }
  };
#pragma unroll
  for (int p = 0; p < NST - 1; ++p)
    if (p < n_tiles) issue(p, p);
  if constexpr (!SYM && !RING) {
    if (a.rope) {
      // Rotary positions, rotate-half pairs (c, c + D/2): this lane holds
      // columns c = 16ks + 8lh + e, whose partners sit in qf[ks + KS_QK/2].
      // The angle of pair c is p * base^(-2c/D) (revolutions in float64).
      const double p = (double)rho + (double)dil * (double)(row0 + lq);
      const double s1 = a.rope_step, s16 = rope_pow(s1, 16);
      double rk = a.rope_rev0 * rope_pow(s1, 8 * lh);
#pragma unroll
      for (int ks = 0; ks < KS_QK / 2; ++ks) {
        double ri = rk;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float f = rope_frac(p, ri);
          const float sn = __builtin_amdgcn_sinf(f), cs = __builtin_amdgcn_cosf(f);
          const float x = (float)qf[ks][e], y = (float)qf[ks + KS_QK / 2][e];
          qf[ks][e] = (__bf16)(x * cs - y * sn);
          qf[ks + KS_QK / 2][e] = (__bf16)(y * cs + x * sn);
          ri *= s1;
        }
        rk *= s16;
      }
    }
  }
  // Make the compiler wait for the Q loads here, after the first copies are
  // issued (so the two latencies overlap) and before the tile loop: the copies
  // are invisible to its counter tracking, so a wait for Q placed inside the
  // loop would also stall on later copies.
#pragma unroll
  for (int ks = 0; ks < KS_QK; ++ks) asm volatile("" ::"v"(qf[ks]));
  static_assert(NST >= 2 && NST <= 4, "two to four stages");
  for (int j = 0; j < n_tiles; j += NST) {
    step(j, IntC<0>{});
    if (j + 1 < n_tiles) step(j + 1, IntC<1>{});
    if constexpr (NST > 2)
      if (j + 2 < n_tiles) step(j + 2, IntC<2 % NST>{});
    if constexpr (NST > 3)
      if (j + 3 < n_tiles) step(j + 3, IntC<3 % NST>{});
  }
  if constexpr (MODE == kSymmetric || CSINK)
    if (n_tiles == 0) {  // (workgroup-uniform) no tile step waited for the staged rows
      wait_dma_keep(0);
      __syncthreads();
    }
  // Keys outside the band, one at a time in registers: the few global keys of
  // Longformer mode (at most kValuGlobals) and the sink tokens of causal mode.
  // Each lane holds half of its row's q and forms the other half's partial dot
  // product through the partner lane; the state (m, l, O) is updated as for a
  // tile of one key, with P in fp32.  `take` drops keys the band already
  // counted (and rows past the end).
  // The products run on v_dot2_f32_bf16 straight from the packed bf16 q, k
  // and v (no unpacking); the weight is rounded to bf16 first, as the band's
  // P is, and the row sum takes that rounded weight.
  auto extra_key = [&](const char *kr, const char *vr, bool take) {
    float part = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS_QK; ++ks) {
      const U4 kk = *reinterpret_cast<const U4 *>(kr + (ks * 16 + lh * 8) * 2);
      // (through the U4 struct: indexing a bit-cast ext_vector of uint32 here
      // made this compiler read word 0 for every w)
      const U4 qw = __builtin_bit_cast(U4, qf[ks]);
#pragma unroll
      for (int w = 0; w < 4; ++w)
        part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qw.w[w]),
                                               __builtin_bit_cast(bf16x2, kk.w[w]), part, false);
    }
    const float dot = xhalf_add(part);
    rescale(take ? dot : -INFINITY);
    const __bf16 pb = (__bf16)(take ? __builtin_amdgcn_exp2f(fmaf(dot, a.sl2, -m_use)) : 0.f);
    if (lh == 0) l_run += (float)pb;  // l_run holds per-lane shares until the epilogue
    const bf16x2 p_lo = {pb, (__bf16)0.f}, p_hi = {(__bf16)0.f, pb};
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const uint2 vv = *reinterpret_cast<const uint2 *>(vr + (db * 32 + 8 * g4 + 4 * lh) * 2);
        const bf16x2 v0 = __builtin_bit_cast(bf16x2, vv.x), v1 = __builtin_bit_cast(bf16x2, vv.y);
        acc_o[db][4 * g4 + 0] = __builtin_amdgcn_fdot2_f32_bf16(v0, p_lo, acc_o[db][4 * g4 + 0], false);
        acc_o[db][4 * g4 + 1] = __builtin_amdgcn_fdot2_f32_bf16(v0, p_hi, acc_o[db][4 * g4 + 1], false);
        acc_o[db][4 * g4 + 2] = __builtin_amdgcn_fdot2_f32_bf16(v1, p_lo, acc_o[db][4 * g4 + 2], false);
        acc_o[db][4 * g4 + 3] = __builtin_amdgcn_fdot2_f32_bf16(v1, p_hi, acc_o[db][4 * g4 + 3], false);
      }
  };
  if constexpr (MODE == kSymmetric) {
    // global keys; one already inside the row's (dilated) window is skipped
    if (a.G > 0 && has_rows) {
      for (int u = 0; u < a.G; ++u) {
        // g is in the dilated window of row rho + dil*my_row iff it lies in
        // the row's residue class (a wave-uniform test) at class index c
        // with |my_row - c| <= r
        const int dg = uni(gl.idx[b * a.G + u] - rho);
        const bool same_class = dg % dil == 0;
        const int c = dg / dil;
        const bool in_win = same_class && my_row - c <= a.W && c - my_row <= a.W;
        extra_key(gkv + u * Gm::ROWB, gkv + (kValuGlobals + u) * Gm::ROWB,
                  my_row < n_cls && !in_win);
      }
    }
  }
  if constexpr (CSINK) {
    // sink tokens s < n_sink before the row's window (s <= t - W); those
    // inside it were counted by the band
    if (has_rows)
      for (int sk = 0; sk < n_sink; ++sk)
        extra_key(gkv + sk * Gm::ROWB, gkv + (kMaxSinks + sk) * Gm::ROWB,
                  my_row < n_cls && sk <= my_row - a.W);
  }
  // global rows: start this wave's loads now (see gp_load)
  GlobalPart<D> gpart;
  const bool gp_on = SYM && a.gws != nullptr && row0 < n_cls;
  if constexpr (SYM)
    if (gp_on) gp_load<D, GPROJ>(gpart, a, gl, b, h, kvh, rho, dil, n_cls, row0);
  // other waves may still read the last stage, which the output staging reuses
  lds_barrier();

  // -------- epilogue: normalise, stage rows through LDS, coalesced stores
  // With a sink score z (natural-log units) the denominator gains exp(z): in
  // the log2 domain of m, l that is 2^(z log2 e - m), taken against the larger
  // of m and z log2 e so neither side overflows.
  l_run = xhalf_add(l_run);  // the two half-waves' key shares of each row
  float inv_l = (l_run > 0.f) ? 1.f / l_run : 0.f;
  float lse_l2 = (l_run > 0.f) ? m_run + __log2f(l_run) : -INFINITY;  // log2 units
  if (SCORE && a.sink_logit) {
    const float z2 = a.sink_logit[h] * 1.4426950408889634f;
    const float mu = (m_run == -INFINITY) ? z2 : fmaxf(m_run, z2);
    const float sc = (l_run > 0.f) ? __builtin_amdgcn_exp2f(m_run - mu) : 0.f;
    const float lt = l_run * sc + __builtin_amdgcn_exp2f(z2 - mu);
    inv_l = sc / lt;
    lse_l2 = mu + __log2f(lt);
  }
  // Each wave stages its 32 rows (row-major, 16-byte chunks XOR-swizzled by
  // row, no padding) in its own slice of the now idle stage memory.
  uint16_t *ost = reinterpret_cast<uint16_t *>(smem + wave * kRowsPerWave * D * 2);
  constexpr int CPRo = D / 8;  // 16-byte chunks per staged row
  auto ost_off = [&](int row, int col) {  // element offset of (row, col)
    return row * D + ((((col >> 3) ^ (row & (CPRo - 1))) << 3) | (col & 7));
  };
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d = db * 32 + 8 * g4 + 4 * lh;
      uint2 w;
      w.x = pack_bf16(acc_o[db][4 * g4 + 0] * inv_l, acc_o[db][4 * g4 + 1] * inv_l);
      w.y = pack_bf16(acc_o[db][4 * g4 + 2] * inv_l, acc_o[db][4 * g4 + 3] * inv_l);
      *reinterpret_cast<uint2 *>(ost + ost_off(lq, d)) = w;
    }
  if (a.lse && lh == 0 && my_row < n_cls) {
    const long long t_abs = rho + (long long)dil * my_row;
    const float lse = lse_l2 * 0.69314718055994531f;
    a.lse[((long long)b * a.Hq + h) * a.T + t_abs] = lse;
  }
  lds_barrier();
  uint16_t *og = static_cast<uint16_t *>(a.o);
  constexpr int LPR = D / 8;             // lanes per row (16 B each)
  constexpr int RPI = 64 / LPR;          // rows per wave instruction
#pragma unroll
  for (int it = 0; it < kRowsPerWave / RPI; ++it) {
    const int rr = it * RPI + lane / LPR;
    const int c = lane % LPR;
    const int r = row0 + rr;
    if (r < n_cls) {
      const U4 u = *reinterpret_cast<const U4 *>(ost + ost_off(rr, c * 8));
      const long long t_abs = rho + (long long)dil * r;
      // written once, never read here: a non-temporal store, so the output
      // rows do not push the key/value band out of L2
      __builtin_nontemporal_store(__builtin_bit_cast(u32x4, u),
                                  reinterpret_cast<u32x4 *>(og + (long long)b * a.q_sb + t_abs * a.q_st + (long long)h * D + c * 8));
    }
  }

  // -------- global rows: partial over this wave's 32 keys
  if constexpr (SYM)
    if (gp_on) gp_finish<D, GPROJ>(gpart, a, gl, smem + wave * kRowsPerWave * D * 2, b, h, rho, dil, n_cls, row0);
}

// Global rows: merge the per-block states of launch_fwd_bf16's symmetric pass.
// With M = max m_k (log2 units): o = sum_k 2^(m_k - M) O_k / sum_k 2^(m_k - M) l_k,
// lse = (M + log2 L) ln 2.  A record's D outputs are read as D/4 float4 by as
// many lanes, so one pass of the workgroup covers 1024/D records and all its
// loads are independent.
template <int D>
__global__ __launch_bounds__(256) void global_combine_kernel(const FwdArgs a, const GlobalList gl) {
  constexpr int PS = D + 4;      // floats per record
  constexpr int LPR = D / 4;     // lanes per record
  constexpr int RPP = 256 / LPR; // records per pass
  __shared__ float s_m[RPP];
  __shared__ float s_l[RPP];
  __shared__ float4 s_o[RPP][LPR];
  const int u = group_x(), h = group_y(), b = group_z();
  const int tid = thread_x();
  const int c = tid % LPR, j = tid / LPR;
  const int nb = class_tiles(a.T, a.dil[h], kRowsPerWave);
  const float *ws = a.gws + (((long long)b * a.Hq + h) * a.G + u) * a.gnb * PS;
  // One pass: thread (j, c) merges records j, j + RPP, ... (float4 c of each)
  // against the largest of their maxima, then the RPP partial states merge in
  // LDS against the overall maximum.  Every record load is independent.
  constexpr int KMAX = 8;  // records per thread held at once
  float mj = -INFINITY, L = 0.f;
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int k0 = j; k0 < nb; k0 += KMAX * RPP) {
    float2 ml[KMAX];
    float4 x[KMAX];
#pragma unroll
    for (int i = 0; i < KMAX; ++i) {
      const int k = min(k0 + i * RPP, nb - 1);  // past the end: a repeat, weight 0
      const float *rec = ws + (long long)k * PS;
      ml[i] = *reinterpret_cast<const float2 *>(rec + D);
      x[i] = *reinterpret_cast<const float4 *>(rec + 4 * c);
    }
    float mn = mj;
#pragma unroll
    for (int i = 0; i < KMAX; ++i)
      if (k0 + i * RPP < nb) mn = fmaxf(mn, ml[i].x);
    if (mn > -INFINITY) {
      const float r = mj > -INFINITY ? __builtin_amdgcn_exp2f(mj - mn) : 0.f;
      L *= r;
      o.x *= r;
      o.y *= r;
      o.z *= r;
      o.w *= r;
#pragma unroll
      for (int i = 0; i < KMAX; ++i) {
        const float sc = (k0 + i * RPP < nb && ml[i].x > -INFINITY) ? __builtin_amdgcn_exp2f(ml[i].x - mn) : 0.f;
        L = fmaf(sc, ml[i].y, L);
        o.x = fmaf(sc, x[i].x, o.x);
        o.y = fmaf(sc, x[i].y, o.y);
        o.z = fmaf(sc, x[i].z, o.z);
        o.w = fmaf(sc, x[i].w, o.w);
      }
      mj = mn;
    }
  }
  if (c == 0) s_m[j] = mj;
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int i = 0; i < RPP; ++i) M = fmaxf(M, s_m[i]);
  const float sj = mj > -INFINITY ? __builtin_amdgcn_exp2f(mj - M) : 0.f;
  o.x *= sj;
  o.y *= sj;
  o.z *= sj;
  o.w *= sj;
  s_o[j][c] = o;
  if (c == 0) s_l[j] = L * sj;
  __syncthreads();
  if (tid < D) {
    float Lt = 0.f, ot = 0.f;
#pragma unroll
    for (int i = 0; i < RPP; ++i) {
      Lt += s_l[i];
      ot += reinterpret_cast<const float *>(&s_o[i][0])[tid];
    }
    const long long pos = gl.idx[b * a.G + u];
    const __bf16 hv = (__bf16)(Lt > 0.f ? ot / Lt : 0.f);
    static_cast<uint16_t *>(a.o)[(long long)b * a.q_sb + pos * a.q_st + (long long)h * D + tid] =
        __builtin_bit_cast(uint16_t, hv);
    if (a.lse && tid == 0)
      a.lse[((long long)b * a.Hq + h) * a.T + pos] =
          Lt > 0.f ? (M + __log2f(Lt)) * 0.69314718055994531f : -INFINITY;
  }
}

}  // namespace

hipError_t launch_global_combine(const FwdArgs &a, int D, const GlobalList *gl, hipStream_t st) {
  const dim3 grid(a.G, a.Hq, a.B);
  if (D == 128) hipLaunchKernelGGL((global_combine_kernel<128>), grid, dim3(256), 0, st, a, *gl);
  else hipLaunchKernelGGL((global_combine_kernel<64>), grid, dim3(256), 0, st, a, *gl);
  return hipGetLastError();
}

hipError_t launch_fwd_bf16(const FwdArgs &a, int mode, int D, const GlobalList *gl,
                           hipStream_t st) {
  const bool sym = mode == kSymmetric || mode == kSymmetricProj;
  int nblk = (sym || mode == kCausalDil) ? a.B * a.tiles_per_batch : a.B * a.n_hg * a.n_qt;
  if (nblk <= 0) return hipSuccess;
  if (mode == kCausalDil) {  // 8 work-balanced XCD ranges
    int most = 0;
    for (int x = 0; x < 8; ++x) most = std::max(most, a.xcd_off[x + 1] - a.xcd_off[x]);
    nblk = 8 * most;
  }
  constexpr int NWC = kFwdWaves;
  if (a.NW != kFwdWaves) return hipErrorInvalidValue;
  dim3 grid(nblk), block(64 * a.NW);
  if (mode == kCausal) {
    if (D == 128) hipLaunchKernelGGL((fwd_kernel<128, kCausal, NWC>), grid, block, 0, st, a, *gl);
    else hipLaunchKernelGGL((fwd_kernel<64, kCausal, NWC>), grid, block, 0, st, a, *gl);
  } else if (mode == kCausalSink) {
    if (D == 128) hipLaunchKernelGGL((fwd_kernel<128, kCausalSink, NWC>), grid, block, 0, st, a, *gl);
    else hipLaunchKernelGGL((fwd_kernel<64, kCausalSink, NWC>), grid, block, 0, st, a, *gl);
  } else if (mode == kRing) {
    if (D == 128) hipLaunchKernelGGL((fwd_kernel<128, kRing, NWC>), grid, block, 0, st, a, *gl);
    else hipLaunchKernelGGL((fwd_kernel<64, kRing, NWC>), grid, block, 0, st, a, *gl);
  } else if (mode == kSymmetricProj) {
    if (D == 128) hipLaunchKernelGGL((fwd_kernel<128, kSymmetricProj, 4>), grid, block, 0, st, a, *gl);
    else hipLaunchKernelGGL((fwd_kernel<64, kSymmetricProj, 4>), grid, block, 0, st, a, *gl);
  } else if (mode == kCausalDil) {
    if (D == 128) hipLaunchKernelGGL((fwd_kernel<128, kCausalDil, NWC>), grid, block, 0, st, a, *gl);
    else hipLaunchKernelGGL((fwd_kernel<64, kCausalDil, NWC>), grid, block, 0, st, a, *gl);
  } else {
    if (D == 128) hipLaunchKernelGGL((fwd_kernel<128, kSymmetric, 4>), grid, block, 0, st, a, *gl);
    else hipLaunchKernelGGL((fwd_kernel<64, kSymmetric, 4>), grid, block, 0, st, a, *gl);
  }
  return hipGetLastError();
}

}  // namespace swa
