// swa_internal.h — definitions shared by the host launchers and the gfx950 kernels.
//
// The row key bounds and the band-tile schedule are written once here as
// __host__ __device__ functions: the banded kernels run them, swa_band_tiles
// exports the schedule and swa_debug_index_mask evaluates the bounds for
// testing.  (The kernels' tile-level mask arithmetic on top of the bounds is
// read out through the kernels themselves by the tests.)
//
// Page tags used in comments:
//   [KB] "Sliding Window Attention", LLM architecture knowledge base (lizeman.github.io)
//   [G3] "Sliding Window Attention — Gemma 3" study note (ai-engineer-exhaustive.pages.dev)
//   [PP] "Sliding Window Attention: From Local Windows to Global Context" (prathamp.com)
//   [ST] "Sliding Window Attention (SWA)" glossary (superteams.ai)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/swa.h"

namespace swa {

// Work-item and workgroup ids read straight from the hardware.  The threadIdx,
// blockIdx and blockDim accessors go through device-library functions that
// kernels built with -mno-amdgpu-ieee cannot inline, so each use would be a
// call (whose entry waits for every outstanding memory operation).
__device__ inline int thread_x() { return (int)__builtin_amdgcn_workitem_id_x(); }
__device__ inline int group_x() { return (int)__builtin_amdgcn_workgroup_id_x(); }
__device__ inline int group_y() { return (int)__builtin_amdgcn_workgroup_id_y(); }
__device__ inline int group_z() { return (int)__builtin_amdgcn_workgroup_id_z(); }
__device__ inline int group_size_x() { return (int)__builtin_amdgcn_workgroup_size_x(); }

// ---------------------------------------------------------------- predicates

// Causal window ([KB] §2 N_t, §3 mask): key s is attended by query t iff t-W < s <= t.
__host__ __device__ inline bool causal_in(int t, int s, int W) { return s <= t && s > t - W; }

// Undilated symmetric window in one residue class ([PP] §1.1): |i - j| <= r.
__host__ __device__ inline bool sym_in(int i, int j, int r) {
  const int d = i - j;
  return d <= r && -d <= r;
}

// Dilated window on original positions ([PP] §3.1): j = i + k*dil with |k| <= r.
__host__ __device__ inline bool dilated_in(int i, int j, int r, int dil) {
  const int d = i - j;
  if (d % dil != 0) return false;
  const int k = d / dil;
  return k <= r && -k <= r;
}

// Attended keys of one row as an interval in the banded kernels' index space:
// causal row t of a sequence of n keys attends [t-W+1, min(t, n-1)] ([KB] §2
// N_t, cut at 0 by the key range); row i of one residue class of length n
// attends [i-r, min(i+r, n-1)] ([PP] §1.1 inside the class, §3.1).  The banded
// kernel masks its partial tiles by comparing key indices with these bounds;
// swa_debug_index_mask evaluates the same bounds (and the same class mapping)
// for every (row, key) pair.
__host__ __device__ inline void row_key_bounds(bool symmetric, int i, int w_or_r, int n, int *lo,
                                               int *hi) {
  *lo = symmetric ? i - w_or_r : i - w_or_r + 1;
  const int h = symmetric ? (i >= n - 1 - w_or_r ? n - 1 : i + w_or_r) : i;  // no overflow
  *hi = h < n - 1 ? h : n - 1;
}

// ---------------------------------------------------------------- band tiles
//
// A query tile holds the valid rows [t0, t1]; key tiles have BN columns.  The
// visited key tiles form the contiguous range [lo, hi] (every tile in it holds
// at least one attended pair); a visited tile needs a mask unless every pair
// of valid rows x columns in it is attended (columns >= n count as masked).

struct TileRange {
  int lo, hi;
};

__host__ __device__ inline TileRange causal_tile_range(int t0, int t1, int W, int BN) {
  int s_lo = t0 - W + 1;
  if (s_lo < 0) s_lo = 0;
  return {s_lo / BN, t1 / BN};
}

// The tiles needing no mask are a contiguous range too (empty when lo > hi):
// tile kj (columns s0 = kj*BN .. s1 = s0+BN-1) is full iff s1 <= t0 (every
// column at or before the first row), s0 > t1 - W (inside the last row's
// window) and s1 < n.
__host__ __device__ inline TileRange causal_full_range(int t0, int t1, int W, int BN, int n) {
  const int x = t1 - W + 1;  // first column of the last row's window
  const int lo = x <= 0 ? 0 : (x + BN - 1) / BN;
  const int hi = ((t0 + 1 < n ? t0 + 1 : n) / BN) - 1;
  return {lo, hi};
}

__host__ __device__ inline bool causal_tile_full(int t0, int t1, int kj, int BN, int W, int n) {
  const TileRange f = causal_full_range(t0, t1, W, BN, n);
  return kj >= f.lo && kj <= f.hi;
}

__host__ __device__ inline TileRange sym_tile_range(int i0, int i1, int r, int n, int BN) {
  int s_lo = i0 - r;
  if (s_lo < 0) s_lo = 0;
  const int s_hi = i1 >= n - 1 - r ? n - 1 : i1 + r;  // no overflow for large r
  return {s_lo / BN, s_hi / BN};
}

// Full tiles: s1 - i0 <= r, i1 - s0 <= r and s1 < n (empty when lo > hi).
__host__ __device__ inline TileRange sym_full_range(int i0, int i1, int r, int BN, int n) {
  const int x = i1 - r;  // first column within r of the last row
  const int lo = x <= 0 ? 0 : (x + BN - 1) / BN;
  const int top = i0 >= n - 1 - r ? n : i0 + r + 1;  // one past the first row's last column
  return {lo, top / BN - 1};
}

__host__ __device__ inline bool sym_tile_full(int i0, int i1, int kj, int BN, int r, int n) {
  const TileRange f = sym_full_range(i0, i1, r, BN, n);
  return kj >= f.lo && kj <= f.hi;
}

// ---------------------------------------------------------------- residue classes
//
// A head with dilation dil splits positions into dil classes rho = i mod dil;
// within a class the dilated window is an undilated window of radius r on the
// subsequence rho, rho+dil, ... ([PP] §3.1-3.2: keys i + k*dil stay in i's class).
struct ClassSplit {
  int q, rem;  // n = q*dil + rem; classes rho < rem have length q+1, others q
};
__host__ __device__ inline ClassSplit class_split(int n, int dil) { return {n / dil, n % dil}; }
__host__ __device__ inline int class_len(ClassSplit c, int rho) { return c.q + (rho < c.rem ? 1 : 0); }
__host__ __device__ inline int ceil_div(int a, int b) { return (a + b - 1) / b; }
// Number of BM-row query tiles a head with dilation dil needs over all its classes.
__host__ __device__ inline int class_tiles(int n, int dil, int BM) {
  const ClassSplit c = class_split(n, dil);
  return c.rem * ceil_div(c.q + 1, BM) + (dil - c.rem) * ceil_div(c.q, BM);
}
// First tile index of class rho in the enumeration above (classes in order).
__host__ __device__ inline int class_tile_base(int n, int dil, int BM, int rho) {
  const ClassSplit c = class_split(n, dil);
  const int c1 = ceil_div(c.q + 1, BM), c0 = ceil_div(c.q, BM);
  return rho < c.rem ? rho * c1 : c.rem * c1 + (rho - c.rem) * c0;
}
// Inverse of the enumeration above: tile index -> (class, tile within class).
__host__ __device__ inline void class_tile_decode(int n, int dil, int BM, int idx, int *rho, int *tile) {
  const ClassSplit c = class_split(n, dil);
  const int c1 = ceil_div(c.q + 1, BM), c0 = ceil_div(c.q, BM);
  if (idx < c.rem * c1) {
    *rho = idx / c1;
    *tile = idx % c1;
  } else {
    idx -= c.rem * c1;
    *rho = c.rem + idx / c0;
    *tile = idx % c0;
  }
}

// ---------------------------------------------------------------- launch geometry

// Consecutive workgroup ids are dispatched round-robin over the 8 XCDs, each
// with its own L2.  Remap so that every XCD owns one contiguous range of
// logical ids (neighbouring query tiles of the same head share K/V in that L2).
__device__ inline int xcd_remap(int bid, int nblocks) {
  constexpr int NX = 8;
  const int q = nblocks / NX, rem = nblocks % NX;
  const int x = bid % NX, idx = bid / NX;
  return x * q + (x < rem ? x : rem) + idx;
}

// Key tile (columns) of the bf16 MFMA kernels: 32 keys at d_h = 128, 64 at
// d_h = 64 (8 KB of K per tile either way).
__host__ __device__ constexpr int key_tile(int D) { return D == 64 ? 64 : 32; }
constexpr int kRowsPerWave = 32; // query rows per wave (one 32x32 MFMA block)

// Waves per workgroup of the bf16 banded kernels: four, one per SIMD, with
// three workgroups per CU at the causal kernels' register count.  Every wave
// of a workgroup reads the same staged K/V tiles, so larger workgroups would
// copy fewer bytes into LDS per FLOP, but their waves share SIMDs behind one
// barrier per tile and ran slower.
constexpr int kFwdWaves = 4;


// Heads packed into one workgroup for the causal kernel: waves of one
// workgroup take query heads that share a key/value head, so a staged K/V tile
// serves several heads ([ST] "Combining SWA with GQA": query heads share one
// key/value head).
inline int prefill_pack(int H_q, int H_kv) {
  const int g = H_q / H_kv;
  return (g % 4 == 0) ? 4 : (g % 2 == 0) ? 2 : 1;
}

// ---------------------------------------------------------------- rotary positions
//
// Revolutions of the RoPE angle for pair i at position p: p * rev0 * step^i with
// rev0 = 1 / 2pi and step = base^(-2/D), in float64 (fp32 would lose ~1e-3 rad
// at positions ~1e4); step^i by binary powering.  Returned as the fraction in
// [0, 1), the argument the sine/cosine units take.
__host__ __device__ inline double rope_pow(double step, int i) {
  double r = 1.0, s = step;
  for (; i > 0; i >>= 1, s *= s)
    if (i & 1) r *= s;
  return r;
}
__host__ __device__ inline float rope_frac(double p, double rev_i) {
  const double x = p * rev_i;
  return (float)(x - floor(x));
}

// ---------------------------------------------------------------- kernel arguments

constexpr int kMaxHeadsLF = 256;
constexpr int kMaxGlobalsLF = 512;

struct FwdArgs {
  const void *q, *k, *v;
  void *o;
  float *lse;
  int B, T, Hq, Hkv;
  long long q_sb, q_st;  // element strides of q/o: batch, token (head stride = D)
  long long k_sb, k_st;  // element strides of k/v: batch, key row
  long long k_sh;        // element stride of k/v heads (d_h for [B, T, H, d_h])
  int W;                 // causal window, or radius r in symmetric mode
  float sl2;             // scale * log2(e)
  int P, group;          // heads per workgroup, H_q / H_kv
  int n_qt, n_hg;        // causal: query tiles per head group, head groups
  int BM;                // query rows per workgroup
  int NW;                // waves per workgroup
  // symmetric (Longformer) and dilated causal modes: work is enumerated per
  // head (symmetric) or head group of P heads (dilated causal), residue class
  // and query tile
  int G;                       // globals per batch row
  int tiles_per_batch;         // sum over heads / head groups of class tiles
  int head_off[kMaxHeadsLF + 1];   // prefix sums of class tiles per head (group)
  unsigned short dil[kMaxHeadsLF]; // dilation per head (group)
  // ring mode (a chunk of queries over a ring cache)
  const int *slot_pos;   // [B, S] position held by each slot (< 0 = empty)
  const int *q_pos;      // [B, T] absolute position of each query row
  int S;                 // ring slots (key rows per batch and head)
  // attention sinks (causal and ring modes)
  int n_sink;                // the first n_sink positions stay visible (<= kMaxSinks)
  const float *sink_logit;   // [H_q] per-head sink score in the denominator, or null
  // symmetric mode: separate global projections (null = shared with q, k, v)
  const void *qg, *kg, *vg;
  // symmetric mode, global rows (bf16): partial softmax states of every global
  // row over each 32-key block of class positions, [B][H][G][gnb] records of
  // D + 4 floats (D unnormalised outputs, m in log2 units, l); null = the
  // global rows are computed by the split-KV pass instead
  float *gws;
  int gnb;  // record slots per (batch, head, global row): max over heads of the blocks
  // rotary positions applied to q in registers (causal modes): the pair
  // (x_i, x_{i+D/2}) of a row at position p turns by p * rope_rev0 * rope_step^i
  // revolutions (rope_rev0 = 1 / 2pi, rope_step = base^(-2/D))
  int rope;
  double rope_rev0, rope_step;
  // dilated causal mode: XCD x runs the work items [xcd_off[x], xcd_off[x+1])
  // of the enumeration (ranges cut for equal work, see dilated_xcd_ranges);
  // the grid is 8 * the longest range
  int xcd_off[9];
};

constexpr int kMaxSinks = 32;  // few: the causal kernel adds them one key at a time
// Longformer mode: up to this many global tokens per row the banded kernel adds
// the global keys after the band in registers; more take a tile of global keys.
constexpr int kValuGlobals = 32;

// Window families of the banded kernels (kCausalSink: causal plus attention
// sinks, a separate instantiation so the plain causal kernel carries none of it).
// kSymmetricProj: symmetric with separate global projections.  kCausalDil:
// causal with a dilation per head group (residue classes, like symmetric mode).
enum FwdMode {
  kCausal = 0,
  kSymmetric = 1,
  kRing = 2,
  kCausalSink = 3,
  kSymmetricProj = 4,
  kCausalDil = 5
};


struct GlobalList {
  int idx[kMaxGlobalsLF];  // [B][G] positions
};

// Split-KV attention for few queries against many keys (ring decode, and the
// global rows of Longformer attention, which attend every position).
struct SplitArgs {
  const void *q, *k, *v;
  void *o;
  float *lse;
  float *ws;  // partials: [B][NH][NQ][S] x (D acc, m, l)
  const int *slot_pos, *cur_pos;  // decode mode
  int B, NKV, NQ;        // batch, key/value heads, queries per kv head
  int n_keys, chunk, S;  // keys per (b, kv head), keys per split, splits
  int W;                 // decode window
  long long q_sb, q_sh, q_sq;     // q strides: batch, kv head, query-in-group
  long long k_sb, k_sh, k_sr;     // k/v strides: batch, head, key row
  long long o_sb, o_sh, o_sq;     // o strides
  float sl2;
  int merge;  // bf16: the S splits are the waves of one workgroup (S in {1, 2, 4, 8})
};

// ---------------------------------------------------------------- launchers (host)

hipError_t launch_fwd_bf16(const FwdArgs &a, int mode, int D, const GlobalList *gl,
                           hipStream_t st);
// Merges the per-block partial states of the global rows (FwdArgs::gws) into
// their output rows and lse.
hipError_t launch_global_combine(const FwdArgs &a, int D, const GlobalList *gl, hipStream_t st);
hipError_t launch_fwd_f32(const FwdArgs &a, int mode, int D, const GlobalList *gl,
                          hipStream_t st);
hipError_t launch_split(const SplitArgs &a, bool decode, bool f32, int D, const GlobalList *gl,
                        int G, int H, hipStream_t st);
int mfma_qg(int nq);  // queries per pass of the bf16 split kernel
hipError_t launch_cache_write(bool f32, const void *kn, const void *vn, const int *pos, void *kc,
                              void *vc, int *slot_pos, int B, int L, int S, int Hkv, int D,
                              int n_sink, hipStream_t st);
hipError_t launch_rope(bool f32, const void *x, void *y, const int *pos, int B, int T, int H, int D,
                       double rev0, double step, hipStream_t st);
hipError_t launch_debug_mask(int mode, int T, int w_or_r, int dil, const GlobalList *gl, int G,
                             uint8_t *mask, hipStream_t st);

}  // namespace swa
