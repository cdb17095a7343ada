// swa_api.hip — the C ABI of libswa.so (declared in include/swa.h).
//
// Every entry point validates all arguments on the host, then launches the
// gfx950 kernels asynchronously on the caller's stream.  Nothing is allocated
// and no state is kept between calls, apart from the per-GPU scratch array of
// swa_decode_noalloc and its cached device addresses.
//
// Tags: [KB] knowledge-base page "Sliding Window Attention" (lizeman.github.io);
// [G3] "Sliding Window Attention — Gemma 3" study note (ai-engineer-exhaustive);
// [PP] "Sliding Window Attention: From Local Windows to Global Context" (prathamp.com);
// [ST] "Sliding Window Attention (SWA)" glossary (superteams.ai).

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>
#include <vector>

#include "swa_internal.h"

namespace swa {

int split_max_chunk();

namespace {

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
bool dt_ok(swa_dtype dt) { return dt == SWA_BF16 || dt == SWA_F32; }
bool d_ok(int d) { return d == 64 || d == 128; }
bool scale_ok(float s) { return std::isfinite(s) && s > 0.f; }
constexpr float kLog2e = 1.4426950408889634f;
constexpr double kRev0 = 0.15915494309189535;  // 1 / 2pi: radians -> revolutions

// Number of splits for split-KV over n_keys keys per (batch, head): enough
// workgroups to fill the chip (target), each chunk whole 32-key blocks
// between 64 keys and maxc.
int choose_splits(long long heads_total, int n_keys, int maxc, int target) {
  int s_min = (n_keys + maxc - 1) / maxc;
  int s_max = (n_keys + 63) / 64;
  long long want = (target + heads_total - 1) / heads_total;
  int s = (int)std::max<long long>(s_min, std::min<long long>(want, s_max));
  if (s < 1) s = 1;
  int chunk = (n_keys + s - 1) / s;
  chunk = std::min(maxc, (chunk + 31) / 32 * 32);  // whole 32-key blocks
  return (n_keys + chunk - 1) / chunk;
}

// Keys per split for S splits (whole 32-key blocks, at most maxc).
int split_chunk(int n_keys, int S, int maxc) {
  int chunk = (n_keys + S - 1) / S;
  return std::min(maxc, (chunk + 31) / 32 * 32);
}

// Split policies.  The fp32 kernel keeps a chunk's scores in LDS (at most
// split_max_chunk() keys); the bf16 kernel streams its chunk and has no limit,
// so it takes fewer, longer splits: one round of resident waves.  The fp32
// policy never gives fewer splits, so it sizes the workspace for both.
#ifndef SWA_STREAM_TARGET
#define SWA_STREAM_TARGET 2048
#endif
constexpr int kStreamMaxChunk = 1 << 20;
int splits_for(bool f32, long long heads_total, int n_keys) {
  return f32 ? choose_splits(heads_total, n_keys, split_max_chunk(), 2048)
             : choose_splits(heads_total, n_keys, kStreamMaxChunk, SWA_STREAM_TARGET);
}
int chunk_for(bool f32, int n_keys, int S) {
  return split_chunk(n_keys, S, f32 ? split_max_chunk() : kStreamMaxChunk);
}

swa_status hip_status(hipError_t e) { return e == hipSuccess ? SWA_OK : SWA_ERR_HIP; }

// Longformer global rows on the bf16 path.  Either the banded kernel leaves a
// partial softmax state per (global row, 32-key block of class positions) and
// launch_global_combine merges them, or a split-KV pass recomputes the rows
// from K and V.  The first needs lf_block_bytes and is taken whenever the
// workspace holds it; swa_longformer_workspace_size covers it for every head
// dilation up to kBlockMaxDil.  The second needs only lf_split_bytes.
constexpr int kBlockMaxDil = 16;
size_t lf_split_bytes(int B, int T, int H, int d_h, int G) {
  const int S = splits_for(true, (long long)B * H, T);
  return (size_t)B * H * G * S * (d_h + 2) * sizeof(float);
}
size_t lf_block_bytes(int B, int H, int d_h, int G, int n_blocks) {
  return (size_t)B * H * G * n_blocks * (d_h + 4) * sizeof(float);
}
// Most 32-key blocks any head with dilation <= kBlockMaxDil has.
int lf_block_cap(int T) {
  int m = 0;
  for (int d = 1; d <= kBlockMaxDil; ++d) m = std::max(m, class_tiles(T, d, kRowsPerWave));
  return m;
}

// Dilated causal launch: cut the work items (batch, head group, class, query
// tile; the kernel's enumeration, each class's tiles heaviest first) into 8
// consecutive ranges of equal work, one per XCD.  Work of a tile = the key
// tiles its band visits (causal_tile_range in class index space).
void dilated_xcd_ranges(FwdArgs &a, int BN) {
  std::vector<long long> pre(1, 0);  // prefix sums of work over one batch row
  pre.reserve(a.tiles_per_batch + 1);
  for (int g = 0; g < a.n_hg; ++g) {
    const int dil = a.dil[g];
    const ClassSplit cs = class_split(a.T, dil);
    for (int rho = 0; rho < dil; ++rho) {
      const int n_cls = class_len(cs, rho), nt = ceil_div(n_cls, a.BM);
      for (int i = 0; i < nt; ++i) {
        const int tile = nt - 1 - i;  // heavy first, as the kernel decodes it
        const int t0 = tile * a.BM, t1 = std::min(t0 + a.BM, n_cls) - 1;
        const TileRange tr = causal_tile_range(t0, t1, a.W, BN);
        pre.push_back(pre.back() + (tr.hi - tr.lo + 1));
      }
    }
  }
  const long long per_b = pre.back(), total = per_b * a.B;
  const long long n_items = (long long)a.B * a.tiles_per_batch;
  a.xcd_off[0] = 0;
  for (int x = 1; x < 8; ++x) {
    // first item whose cumulative work reaches x/8 of the total
    const long long target = (total * x + 7) / 8;
    const long long b = target / per_b, rem = target % per_b;
    const long long i = std::lower_bound(pre.begin(), pre.end(), rem) - pre.begin();
    a.xcd_off[x] = (int)std::min(n_items, b * a.tiles_per_batch + i);
  }
  a.xcd_off[8] = (int)n_items;
  for (int x = 1; x <= 8; ++x) a.xcd_off[x] = std::max(a.xcd_off[x], a.xcd_off[x - 1]);
}

}  // namespace
}  // namespace swa

// ---- scratch memory of swa_decode_noalloc -------------------------------------
//
// One array per GPU, in the library's code object: each device that loads the
// library holds its own copy until the process ends.  In host code the name
// `scratch` is only a stand-in; its device address is looked up once per
// device with hipGetSymbolAddress and kept in scratch_addr, and only that
// address ever reaches a kernel.
static __device__ __align__(256) unsigned char scratch[SWA_DECODE_NOALLOC_SCRATCH_BYTES];

namespace swa {
namespace {
constexpr int kMaxDevices = 64;
std::atomic<void *> scratch_addr[kMaxDevices];
std::mutex scratch_mu;

// Device address of the current device's scratch array (looked up on the
// first call on that device).
swa_status scratch_for_current_device(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return SWA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return SWA_ERR_UNSUPPORTED;
  void *p = scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(scratch_mu);
    p = scratch_addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SWA_ERR_HIP;
      scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return SWA_OK;
}
}  // namespace
}  // namespace swa

using namespace swa;

extern "C" {

const char *swa_status_str(swa_status s) {
  switch (s) {
    case SWA_OK: return "ok";
    case SWA_ERR_INVALID: return "invalid argument";
    case SWA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case SWA_ERR_WORKSPACE: return "workspace too small";
    case SWA_ERR_HIP: return "HIP launch error";
  }
  return "unknown status";
}

int swa_version(void) { return 1; }

swa_status swa_tile_config(int entry, int H_q, int H_kv, int d_h, int *BM, int *BN) {
  if (!BM || !BN || H_q < 1 || H_kv < 1 || H_q % H_kv) return SWA_ERR_INVALID;
  if (!d_ok(d_h)) return SWA_ERR_UNSUPPORTED;
  if (entry == 'p') {
    *BM = kRowsPerWave * kFwdWaves / prefill_pack(H_q, H_kv);
  } else if (entry == 'l') {
    *BM = kRowsPerWave * kFwdWaves;
  } else {
    return SWA_ERR_INVALID;
  }
  *BN = key_tile(d_h);
  return SWA_OK;
}

int swa_band_tiles(int mode, int T, int w_or_r, int BM, int BN, int32_t *out, int cap) {
  if (T < 1 || BM < 1 || BN < 1 || cap < 0 || (cap > 0 && !out)) return -1;
  if (mode == SWA_MODE_CAUSAL ? w_or_r < 1 : (mode == SWA_MODE_SYMMETRIC ? w_or_r < 0 : true))
    return -1;
  int n = 0;
  const int nq = (T + BM - 1) / BM;
  for (int qi = 0; qi < nq; ++qi) {
    const int t0 = qi * BM, t1 = std::min(T, t0 + BM) - 1;
    const TileRange tr = mode == SWA_MODE_CAUSAL ? causal_tile_range(t0, t1, w_or_r, BN)
                                                 : sym_tile_range(t0, t1, w_or_r, T, BN);
    for (int kj = tr.lo; kj <= tr.hi; ++kj) {
      const bool full = mode == SWA_MODE_CAUSAL ? causal_tile_full(t0, t1, kj, BN, w_or_r, T)
                                                : sym_tile_full(t0, t1, kj, BN, w_or_r, T);
      if (n < cap) {
        out[3 * n] = qi;
        out[3 * n + 1] = kj;
        out[3 * n + 2] = full ? 0 : 1;
      }
      ++n;
    }
  }
  return n;
}

swa_status swa_prefill(swa_dtype dt, const void *q, const void *k, const void *v, void *o,
                       float *lse, int B, int T, int H_q, int H_kv, int d_h, int W, float scale,
                       void *stream) {
  return swa_prefill_sinks(dt, q, k, v, o, lse, B, T, H_q, H_kv, d_h, W, 0, nullptr, scale,
                           stream);
}

swa_status swa_prefill_sinks(swa_dtype dt, const void *q, const void *k, const void *v, void *o,
                             float *lse, int B, int T, int H_q, int H_kv, int d_h, int W,
                             int n_sink, const float *sink_logit, float scale, void *stream) {
  if (!dt_ok(dt) || !q || !k || !v || !o) return SWA_ERR_INVALID;
  if (n_sink < 0 || n_sink > kMaxSinks || (sink_logit && !aligned(sink_logit, 4)))
    return SWA_ERR_INVALID;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      (lse && !aligned(lse, 4)))
    return SWA_ERR_INVALID;
  if (B < 1 || T < 1 || H_q < 1 || H_kv < 1 || W < 1 || H_q % H_kv || !scale_ok(scale))
    return SWA_ERR_INVALID;
  if (!d_ok(d_h)) return SWA_ERR_UNSUPPORTED;

  FwdArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.B = B; a.T = T; a.Hq = H_q; a.Hkv = H_kv;
  a.q_st = (long long)H_q * d_h;
  a.q_sb = a.q_st * T;
  a.k_st = (long long)H_kv * d_h;
  a.k_sb = a.k_st * T;
  a.k_sh = d_h;
  a.n_sink = n_sink;
  a.sink_logit = sink_logit;
  a.W = W;
  a.sl2 = scale * kLog2e;
  a.group = H_q / H_kv;
  const int mode = (n_sink > 0 || sink_logit) ? kCausalSink : kCausal;
  a.P = prefill_pack(H_q, H_kv);
  a.NW = kFwdWaves;
  a.BM = kRowsPerWave * a.NW / a.P;
  a.n_qt = (T + a.BM - 1) / a.BM;
  a.n_hg = H_q / a.P;
  GlobalList gl;
  std::memset(&gl, 0, sizeof(gl));
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dt == SWA_F32) return hip_status(launch_fwd_f32(a, mode, d_h, &gl, st));
  // bf16 kernels address one batch slice of K/V with 32-bit byte offsets
  if ((long long)B * a.n_hg * a.n_qt > 0x7fffffffLL || a.k_sb * 2 >= (1LL << 31))
    return SWA_ERR_UNSUPPORTED;
  return hip_status(launch_fwd_bf16(a, mode, d_h, &gl, st));
}

swa_status swa_prefill_dilated(swa_dtype dt, const void *q, const void *k, const void *v, void *o,
                               float *lse, int B, int T, int H_q, int H_kv, int d_h, int W,
                               const int32_t *dilation, float scale, void *stream) {
  if (!dt_ok(dt) || !q || !k || !v || !o) return SWA_ERR_INVALID;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      (lse && !aligned(lse, 4)))
    return SWA_ERR_INVALID;
  if (B < 1 || T < 1 || H_q < 1 || H_kv < 1 || W < 1 || H_q % H_kv || !scale_ok(scale))
    return SWA_ERR_INVALID;
  if (dilation)
    for (int h = 0; h < H_q; ++h)
      if (dilation[h] < 1 || dilation[h] > 65535) return SWA_ERR_INVALID;
  if (!d_ok(d_h)) return SWA_ERR_UNSUPPORTED;
  bool any = false;
  for (int h = 0; dilation && h < H_q; ++h) any |= dilation[h] != 1;
  if (!any)
    return swa_prefill(dt, q, k, v, o, lse, B, T, H_q, H_kv, d_h, W, scale, stream);

  FwdArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.B = B; a.T = T; a.Hq = H_q; a.Hkv = H_kv;
  a.q_st = (long long)H_q * d_h;
  a.q_sb = a.q_st * T;
  a.k_st = (long long)H_kv * d_h;
  a.k_sb = a.k_st * T;
  a.k_sh = d_h;
  a.W = W;
  a.sl2 = scale * kLog2e;
  a.group = H_q / H_kv;
  GlobalList gl;
  std::memset(&gl, 0, sizeof(gl));
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dt == SWA_F32) {
    if (H_q > kMaxHeadsLF) return SWA_ERR_UNSUPPORTED;
    for (int h = 0; h < H_q; ++h) a.dil[h] = (unsigned short)dilation[h];
    return hip_status(launch_fwd_f32(a, kCausalDil, d_h, &gl, st));
  }
  // Heads packed into one workgroup share their key/value head; they must
  // share the dilation too, else one head per workgroup.
  int P = prefill_pack(H_q, H_kv);
  for (int h = 0; h < H_q && P > 1; ++h)
    if (dilation[h] != dilation[h - h % P]) P = 1;
  a.P = P;
  a.NW = kFwdWaves;
  a.BM = kRowsPerWave * a.NW / P;
  a.n_hg = H_q / P;
  if (a.n_hg > kMaxHeadsLF) return SWA_ERR_UNSUPPORTED;
  long long tiles = 0;
  for (int g = 0; g < a.n_hg; ++g) {
    a.dil[g] = (unsigned short)dilation[g * P];
    a.head_off[g] = (int)tiles;
    tiles += class_tiles(T, a.dil[g], a.BM);
  }
  a.head_off[a.n_hg] = (int)tiles;
  // bf16 kernels address one batch slice of K/V with 32-bit byte offsets
  if (tiles * B > 0x7fffffffLL || a.k_sb * 2 >= (1LL << 31)) return SWA_ERR_UNSUPPORTED;
  a.tiles_per_batch = (int)tiles;
  dilated_xcd_ranges(a, key_tile(d_h));
  return hip_status(launch_fwd_bf16(a, kCausalDil, d_h, &gl, st));
}

size_t swa_prefill_rope_workspace_size(swa_dtype dt, int B, int T, int H_kv, int d_h) {
  if (!dt_ok(dt) || B < 1 || T < 1 || H_kv < 1 || !d_ok(d_h)) return 0;
  return (size_t)B * T * H_kv * d_h * (dt == SWA_F32 ? 4 : 2);
}

swa_status swa_rope(swa_dtype dt, const void *x, void *y, const int32_t *pos, int B, int T, int H,
                    int d_h, float rope_base, void *stream) {
  if (!dt_ok(dt) || !x || !y || !aligned(x, 16) || !aligned(y, 16) || (pos && !aligned(pos, 4)))
    return SWA_ERR_INVALID;
  if (B < 1 || T < 1 || H < 1 || !std::isfinite(rope_base) || !(rope_base > 0.f))
    return SWA_ERR_INVALID;
  if (!d_ok(d_h)) return SWA_ERR_UNSUPPORTED;
  return hip_status(launch_rope(dt == SWA_F32, x, y, pos, B, T, H, d_h, kRev0,
                                std::pow((double)rope_base, -2.0 / d_h),
                                static_cast<hipStream_t>(stream)));
}

swa_status swa_prefill_rope(swa_dtype dt, const void *q, const void *k, const void *v, void *o,
                            float *lse, int B, int T, int H_q, int H_kv, int d_h, int W,
                            float rope_base, float scale, void *workspace, size_t workspace_bytes,
                            void *stream) {
  if (!dt_ok(dt) || !q || !k || !v || !o) return SWA_ERR_INVALID;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      (lse && !aligned(lse, 4)))
    return SWA_ERR_INVALID;
  if (B < 1 || T < 1 || H_q < 1 || H_kv < 1 || W < 1 || H_q % H_kv || !scale_ok(scale) ||
      !std::isfinite(rope_base) || !(rope_base > 0.f))
    return SWA_ERR_INVALID;
  if (!d_ok(d_h)) return SWA_ERR_UNSUPPORTED;
  const size_t need = swa_prefill_rope_workspace_size(dt, B, T, H_kv, d_h);
  if (!workspace || workspace_bytes < need) return SWA_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return SWA_ERR_INVALID;

  FwdArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q = q; a.k = workspace; a.v = v; a.o = o; a.lse = lse;
  a.B = B; a.T = T; a.Hq = H_q; a.Hkv = H_kv;
  a.q_st = (long long)H_q * d_h;
  a.q_sb = a.q_st * T;
  a.k_st = (long long)H_kv * d_h;
  a.k_sb = a.k_st * T;
  a.k_sh = d_h;
  a.W = W;
  a.sl2 = scale * kLog2e;
  a.group = H_q / H_kv;
  a.P = prefill_pack(H_q, H_kv);
  a.NW = kFwdWaves;
  a.BM = kRowsPerWave * a.NW / a.P;
  a.n_qt = (T + a.BM - 1) / a.BM;
  a.n_hg = H_q / a.P;
  a.rope = 1;
  a.rope_rev0 = kRev0;
  a.rope_step = std::pow((double)rope_base, -2.0 / d_h);
  GlobalList gl;
  std::memset(&gl, 0, sizeof(gl));
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dt == SWA_BF16 &&
      ((long long)B * a.n_hg * a.n_qt > 0x7fffffffLL || a.k_sb * 2 >= (1LL << 31)))
    return SWA_ERR_UNSUPPORTED;
  // keys: one rotation pass into the workspace; queries: rotated in registers
  // by the prefill kernel
  hipError_t e = launch_rope(dt == SWA_F32, k, workspace, nullptr, B, T, H_kv, d_h, a.rope_rev0,
                             a.rope_step, st);
  if (e != hipSuccess) return SWA_ERR_HIP;
  if (dt == SWA_F32) return hip_status(launch_fwd_f32(a, kCausal, d_h, &gl, st));
  return hip_status(launch_fwd_bf16(a, kCausal, d_h, &gl, st));
}

swa_status swa_prefill_cached(swa_dtype dt, const void *q, const void *k_cache,
                              const void *v_cache, const int32_t *slot_pos, const int32_t *q_pos,
                              void *o, float *lse, int B, int L, int S, int H_q, int H_kv,
                              int d_h, int W, int n_sink, const float *sink_logit, float scale,
                              void *stream) {
  if (!dt_ok(dt) || !q || !k_cache || !v_cache || !slot_pos || !q_pos || !o)
    return SWA_ERR_INVALID;
  if (n_sink < 0 || (sink_logit && !aligned(sink_logit, 4))) return SWA_ERR_INVALID;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(o, 16) ||
      !aligned(slot_pos, 4) || !aligned(q_pos, 4) || (lse && !aligned(lse, 4)))
    return SWA_ERR_INVALID;
  if (B < 1 || L < 1 || S < 1 || H_q < 1 || H_kv < 1 || W < 1 || H_q % H_kv || !scale_ok(scale))
    return SWA_ERR_INVALID;
  if (!d_ok(d_h)) return SWA_ERR_UNSUPPORTED;

  FwdArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q = q; a.k = k_cache; a.v = v_cache; a.o = o; a.lse = lse;
  a.B = B; a.T = L; a.Hq = H_q; a.Hkv = H_kv;
  a.q_st = (long long)H_q * d_h;
  a.q_sb = a.q_st * L;
  a.k_st = d_h;                        // [B, H_kv, S, d_h]: rows of one head are contiguous
  a.k_sh = (long long)S * d_h;
  a.k_sb = a.k_sh * H_kv;
  a.W = W;
  a.sl2 = scale * kLog2e;
  a.group = H_q / H_kv;
  a.P = prefill_pack(H_q, H_kv);
  a.NW = kFwdWaves;
  a.BM = kRowsPerWave * a.NW / a.P;
  a.n_qt = (L + a.BM - 1) / a.BM;
  a.n_hg = H_q / a.P;
  a.slot_pos = slot_pos;
  a.q_pos = q_pos;
  a.S = S;
  a.n_sink = n_sink;
  a.sink_logit = sink_logit;
  GlobalList gl;
  std::memset(&gl, 0, sizeof(gl));
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dt == SWA_F32) return hip_status(launch_fwd_f32(a, kRing, d_h, &gl, st));
  // bf16 kernels address one (batch, head) slice of K/V with 32-bit byte offsets
  if ((long long)B * a.n_hg * a.n_qt > 0x7fffffffLL || a.k_sh * 2 >= (1LL << 31))
    return SWA_ERR_UNSUPPORTED;
  return hip_status(launch_fwd_bf16(a, kRing, d_h, &gl, st));
}

size_t swa_decode_workspace_size(int B, int H_q, int H_kv, int W, int d_h) {
  if (B < 1 || H_q < 1 || H_kv < 1 || W < 1 || H_q % H_kv || !d_ok(d_h)) return 0;
  const int S = splits_for(true, (long long)B * H_kv, W);
  return (size_t)B * H_q * S * (d_h + 2) * sizeof(float);
}

swa_status swa_decode(swa_dtype dt, const void *q, const void *k_cache, const void *v_cache,
                      const int32_t *slot_pos, const int32_t *cur_pos, void *o, float *lse,
                      int B, int W, int H_q, int H_kv, int d_h, float scale, void *workspace,
                      size_t workspace_bytes, void *stream) {
  if (!dt_ok(dt) || !q || !k_cache || !v_cache || !slot_pos || !cur_pos || !o)
    return SWA_ERR_INVALID;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(o, 16) ||
      !aligned(slot_pos, 4) || !aligned(cur_pos, 4) || (lse && !aligned(lse, 4)))
    return SWA_ERR_INVALID;
  if (B < 1 || W < 1 || H_q < 1 || H_kv < 1 || H_q % H_kv || !scale_ok(scale))
    return SWA_ERR_INVALID;
  if (!d_ok(d_h)) return SWA_ERR_UNSUPPORTED;
  const size_t need = swa_decode_workspace_size(B, H_q, H_kv, W, d_h);
  if (!workspace || workspace_bytes < need) return SWA_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return SWA_ERR_INVALID;

  SplitArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q = q; a.k = k_cache; a.v = v_cache; a.o = o; a.lse = lse;
  a.ws = static_cast<float *>(workspace);
  a.slot_pos = slot_pos; a.cur_pos = cur_pos;
  a.B = B; a.NKV = H_kv; a.NQ = H_q / H_kv;
  a.n_keys = W;
  a.S = splits_for(dt == SWA_F32, (long long)B * H_kv, W);
  a.chunk = chunk_for(dt == SWA_F32, W, a.S);
  if (dt == SWA_BF16) {
    // Enough (batch, kv head, query pass) groups: each workgroup takes one
    // group, its waves split the ring and merge in LDS (no combine pass).
    const int qg = mfma_qg(H_q / H_kv);
    const long long groups = (long long)B * H_kv * ((H_q / H_kv + qg - 1) / qg);
    for (int nsw = 1; nsw <= 8; nsw *= 2) {
      if (groups * nsw >= SWA_STREAM_TARGET || nsw == 8) {
        if (groups * nsw >= SWA_STREAM_TARGET / 2) {
          a.merge = 1;
          a.S = nsw;
          a.chunk = (W + nsw - 1) / nsw;
          a.chunk = (a.chunk + 31) / 32 * 32;
        }
        break;
      }
    }
  }
  a.W = W;
  a.q_sq = d_h; a.q_sh = (long long)a.NQ * d_h; a.q_sb = (long long)H_q * d_h;
  a.o_sq = a.q_sq; a.o_sh = a.q_sh; a.o_sb = a.q_sb;
  a.k_sr = d_h; a.k_sh = (long long)W * d_h; a.k_sb = (long long)H_kv * W * d_h;
  a.sl2 = scale * kLog2e;
  GlobalList gl;
  std::memset(&gl, 0, sizeof(gl));
  return hip_status(launch_split(a, true, dt == SWA_F32, d_h, &gl, 0, H_kv,
                                 static_cast<hipStream_t>(stream)));
}

swa_status swa_decode_noalloc(swa_dtype dt, const void *q, const void *k_cache,
                              const void *v_cache, const int32_t *slot_pos,
                              const int32_t *cur_pos, void *o, float *lse, int B, int W, int H_q,
                              int H_kv, int d_h, float scale, void *stream) {
  // the checks of swa_decode, before any HIP call
  if (!dt_ok(dt) || !q || !k_cache || !v_cache || !slot_pos || !cur_pos || !o)
    return SWA_ERR_INVALID;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(o, 16) ||
      !aligned(slot_pos, 4) || !aligned(cur_pos, 4) || (lse && !aligned(lse, 4)))
    return SWA_ERR_INVALID;
  if (B < 1 || W < 1 || H_q < 1 || H_kv < 1 || H_q % H_kv || !scale_ok(scale))
    return SWA_ERR_INVALID;
  if (!d_ok(d_h)) return SWA_ERR_UNSUPPORTED;
  if (swa_decode_workspace_size(B, H_q, H_kv, W, d_h) > SWA_DECODE_NOALLOC_SCRATCH_BYTES)
    return SWA_ERR_WORKSPACE;
  void *ws = nullptr;
  const swa_status st = scratch_for_current_device(&ws);
  if (st != SWA_OK) return st;
  return swa_decode(dt, q, k_cache, v_cache, slot_pos, cur_pos, o, lse, B, W, H_q, H_kv, d_h,
                    scale, ws, SWA_DECODE_NOALLOC_SCRATCH_BYTES, stream);
}

swa_status swa_cache_write(swa_dtype dt, const void *k_new, const void *v_new, const int32_t *pos,
                           void *k_cache, void *v_cache, int32_t *slot_pos, int B, int W, int H_kv,
                           int d_h, void *stream) {
  if (!dt_ok(dt) || !k_new || !v_new || !pos || !k_cache || !v_cache || !slot_pos)
    return SWA_ERR_INVALID;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16) || !aligned(pos, 4) || !aligned(slot_pos, 4))
    return SWA_ERR_INVALID;
  if (B < 1 || W < 1 || H_kv < 1 || B > 65535) return SWA_ERR_INVALID;
  if (!d_ok(d_h)) return SWA_ERR_UNSUPPORTED;
  return hip_status(launch_cache_write(dt == SWA_F32, k_new, v_new, pos, k_cache, v_cache,
                                       slot_pos, B, 1, W, H_kv, d_h, 0,
                                       static_cast<hipStream_t>(stream)));
}

swa_status swa_cache_append(swa_dtype dt, const void *k_new, const void *v_new,
                            const int32_t *pos, void *k_cache, void *v_cache, int32_t *slot_pos,
                            int B, int L, int S, int H_kv, int d_h, int n_sink, void *stream) {
  if (!dt_ok(dt) || !k_new || !v_new || !pos || !k_cache || !v_cache || !slot_pos)
    return SWA_ERR_INVALID;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16) || !aligned(pos, 4) || !aligned(slot_pos, 4))
    return SWA_ERR_INVALID;
  if (B < 1 || L < 1 || S < 1 || L > S || H_kv < 1 || L > 65535 || H_kv > 65535 || B > 65535 ||
      n_sink < 0 || n_sink >= S)
    return SWA_ERR_INVALID;
  if (!d_ok(d_h)) return SWA_ERR_UNSUPPORTED;
  return hip_status(launch_cache_write(dt == SWA_F32, k_new, v_new, pos, k_cache, v_cache,
                                       slot_pos, B, L, S, H_kv, d_h, n_sink,
                                       static_cast<hipStream_t>(stream)));
}

size_t swa_longformer_workspace_size(int B, int T, int H, int d_h, int G) {
  if (B < 1 || T < 1 || H < 1 || G < 0 || !d_ok(d_h)) return 0;
  if (G == 0) return 0;
  return std::max(swa::lf_split_bytes(B, T, H, d_h, G),
                  swa::lf_block_bytes(B, H, d_h, G, swa::lf_block_cap(T)));
}

}  // extern "C"

namespace swa {
namespace {

// Longformer attention; qg, kg, vg null = the shared projections (swa_longformer),
// else the separate global projections of swa_longformer_proj.
swa_status longformer_impl(swa_dtype dt, const void *q, const void *k, const void *v,
                           const void *qg, const void *kg, const void *vg, void *o, float *lse,
                           int B, int T, int H, int d_h, int r, const int32_t *dilation,
                           const int32_t *global_idx, int G, float scale, void *workspace,
                           size_t workspace_bytes, void *stream) {
  if (!dt_ok(dt) || !q || !k || !v || !o) return SWA_ERR_INVALID;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      (lse && !aligned(lse, 4)))
    return SWA_ERR_INVALID;
  const bool proj = qg != nullptr;
  if (proj && (!aligned(qg, 16) || !aligned(kg, 16) || !aligned(vg, 16)))
    return SWA_ERR_INVALID;
  if (B < 1 || T < 1 || H < 1 || r < 0 || G < 0 || !scale_ok(scale)) return SWA_ERR_INVALID;
  if ((G > 0) != (global_idx != nullptr)) return SWA_ERR_INVALID;
  if (dilation)
    for (int h = 0; h < H; ++h)
      if (dilation[h] < 1 || dilation[h] > 65535) return SWA_ERR_INVALID;
  for (int b = 0; b < B && G > 0; ++b)
    for (int g = 0; g < G; ++g) {
      const int x = global_idx[b * G + g];
      if (x < 0 || x >= T || (g > 0 && x <= global_idx[b * G + g - 1])) return SWA_ERR_INVALID;
    }
  if (!d_ok(d_h) || H > kMaxHeadsLF || (long long)B * G > kMaxGlobalsLF) return SWA_ERR_UNSUPPORTED;
  const size_t need = (dt == SWA_F32 || G == 0) ? 0 : lf_split_bytes(B, T, H, d_h, G);
  if (need > 0 && (!workspace || workspace_bytes < need)) return SWA_ERR_WORKSPACE;
  if (need > 0 && !aligned(workspace, 16)) return SWA_ERR_INVALID;

  FwdArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.B = B; a.T = T; a.Hq = H; a.Hkv = H;
  a.q_st = (long long)H * d_h;
  a.q_sb = a.q_st * T;
  a.k_st = a.q_st;
  a.k_sb = a.q_sb;
  a.k_sh = d_h;
  a.W = r;
  a.sl2 = scale * kLog2e;
  a.group = 1;
  a.P = 1;
  a.NW = kFwdWaves;
  a.BM = kRowsPerWave * a.NW;
  a.G = G;
  long long tiles = 0;
  for (int h = 0; h < H; ++h) {
    const int d = dilation ? dilation[h] : 1;
    a.dil[h] = (unsigned short)d;
    a.head_off[h] = (int)tiles;
    tiles += class_tiles(T, d, a.BM);
  }
  a.head_off[H] = (int)tiles;
  if (tiles * B > 0x7fffffffLL || (dt == SWA_BF16 && a.k_sb * 2 >= (1LL << 31)))
    return SWA_ERR_UNSUPPORTED;
  a.tiles_per_batch = (int)tiles;
  // With no global token the separate projections are never read.
  const bool gproj = proj && G > 0;
  if (gproj) {
    a.qg = qg; a.kg = kg; a.vg = vg;
  }
  // Many global tokens: the tile-of-global-keys kernel, which with shared
  // projections reads the global keys from k, v themselves.
  const bool gtile = gproj || G > kValuGlobals;
  if (gtile && !gproj) {
    a.qg = q; a.kg = k; a.vg = v;
  }
  GlobalList gl;
  std::memset(&gl, 0, sizeof(gl));
  for (int i = 0; i < B * G; ++i) gl.idx[i] = global_idx[i];
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dt == SWA_F32)
    return hip_status(launch_fwd_f32(a, gproj ? kSymmetricProj : kSymmetric, d_h, &gl, st));

  if (G > 0) {
    int nb = 0;
    for (int h = 0; h < H; ++h) nb = std::max(nb, class_tiles(T, a.dil[h], kRowsPerWave));
    if (workspace_bytes >= lf_block_bytes(B, H, d_h, G, nb)) {
      a.gws = static_cast<float *>(workspace);
      a.gnb = nb;
    }
  }
  hipError_t e = launch_fwd_bf16(a, gtile ? kSymmetricProj : kSymmetric, d_h, &gl, st);
  if (e != hipSuccess || G == 0) return hip_status(e);
  if (a.gws) return hip_status(launch_global_combine(a, d_h, &gl, st));
  // Global rows attend every position: split-KV over all T keys, written after
  // (stream order) the local pass, replacing those rows.  With separate
  // projections they read qg against kg, vg.
  SplitArgs s;
  std::memset(&s, 0, sizeof(s));
  s.q = gproj ? qg : q;
  s.k = gproj ? kg : k;
  s.v = gproj ? vg : v;
  s.o = o; s.lse = lse;
  s.ws = static_cast<float *>(workspace);
  s.B = B; s.NKV = H; s.NQ = G;
  s.n_keys = T;
  s.S = splits_for(dt == SWA_F32, (long long)B * H, T);
  s.chunk = chunk_for(dt == SWA_F32, T, s.S);
  s.q_sb = a.q_sb; s.q_sh = d_h; s.q_sq = a.q_st;
  s.o_sb = a.q_sb; s.o_sh = d_h; s.o_sq = a.q_st;
  s.k_sb = a.k_sb; s.k_sh = d_h; s.k_sr = a.k_st;
  s.sl2 = a.sl2;
  return hip_status(launch_split(s, false, false, d_h, &gl, G, H, st));
}

}  // namespace
}  // namespace swa

extern "C" {

swa_status swa_longformer(swa_dtype dt, const void *q, const void *k, const void *v, void *o,
                          float *lse, int B, int T, int H, int d_h, int r, const int32_t *dilation,
                          const int32_t *global_idx, int G, float scale, void *workspace,
                          size_t workspace_bytes, void *stream) {
  return longformer_impl(dt, q, k, v, nullptr, nullptr, nullptr, o, lse, B, T, H, d_h, r,
                         dilation, global_idx, G, scale, workspace, workspace_bytes, stream);
}

swa_status swa_longformer_proj(swa_dtype dt, const void *q, const void *k, const void *v,
                               const void *qg, const void *kg, const void *vg, void *o,
                               float *lse, int B, int T, int H, int d_h, int r,
                               const int32_t *dilation, const int32_t *global_idx, int G,
                               float scale, void *workspace, size_t workspace_bytes,
                               void *stream) {
  if (!qg || !kg || !vg) return SWA_ERR_INVALID;
  return longformer_impl(dt, q, k, v, qg, kg, vg, o, lse, B, T, H, d_h, r, dilation, global_idx,
                         G, scale, workspace, workspace_bytes, stream);
}

swa_status swa_debug_index_mask(int mode, int T, int w_or_r, int dil, const int32_t *global_idx,
                                int G, uint8_t *mask_dev, void *stream) {
  if (!mask_dev || T < 1 || G < 0 || (G > 0 && !global_idx)) return SWA_ERR_INVALID;
  if (mode == SWA_MODE_CAUSAL) {
    if (w_or_r < 1 || G != 0) return SWA_ERR_INVALID;
  } else if (mode == SWA_MODE_SYMMETRIC) {
    if (w_or_r < 0 || dil < 1) return SWA_ERR_INVALID;
  } else {
    return SWA_ERR_INVALID;
  }
  if ((long long)T * T > (1LL << 31) || G > kMaxGlobalsLF) return SWA_ERR_UNSUPPORTED;
  GlobalList gl;
  std::memset(&gl, 0, sizeof(gl));
  for (int g = 0; g < G; ++g) {
    if (global_idx[g] < 0 || global_idx[g] >= T) return SWA_ERR_INVALID;
    gl.idx[g] = global_idx[g];
  }
  return hip_status(launch_debug_mask(mode, T, w_or_r, mode == SWA_MODE_CAUSAL ? 1 : dil, &gl, G,
                                      mask_dev, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
