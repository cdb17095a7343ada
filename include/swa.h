/*
 * swa.h — C ABI of libswa.so: sliding-window attention (SWA) forward pass for
 * AMD Instinct MI355X (gfx950).
 *
 * What is computed.  For a query position t with connectivity set S_t,
 *     o_t = sum_{s in S_t} softmax_s(scale * q_t . k_s) v_s
 * (the masked softmax of the "Sliding Window Attention" knowledge-base page
 * (lizeman.github.io/llm-arch-kb), §2 "Derivation", and the common form in §11.1
 * of "Sliding Window Attention: From Local Windows to Global Context"
 * (prathamp.com)).  The entry points differ only in S_t:
 *   swa_prefill     causal window  t-W < s <= t                (knowledge base §2, §3)
 *   swa_prefill_dilated  causal windows {t - i*d : 0 <= i < W} with a dilation
 *                   per head (knowledge base §2 "Dilation")
 *   swa_prefill_sinks  the causal window plus pinned sink tokens and an optional
 *                   per-head sink score (knowledge base §4; superteams.ai "What's New")
 *   swa_decode      ring cache of W slots, window from stored absolute positions
 *                   (knowledge base §2 "KV cache"; "Sliding Window Attention —
 *                   Gemma 3" study note, "How it works")
 *   swa_longformer  symmetric window |i-j| <= r with per-head dilation and
 *                   global tokens (prathamp.com §1.1, §3.1, §4.3)
 *   swa_prefill_cached  a chunk of queries with absolute positions over a ring
 *                   cache of S slots (Gemma 3 note, "How it works": positions
 *                   [B, L] against cache positions [B, S]); swa_decode is the
 *                   one-token case
 *
 * Conventions shared by every entry point.
 *   - Tensors are caller-owned, contiguous, row-major DEVICE buffers unless an
 *     argument says HOST.  Element type: bf16 (SWA_BF16) or float32 (SWA_F32)
 *     for q/k/v/o; lse is always float32; positions are int32.  Device
 *     pointers must be 16-byte aligned.
 *   - d_h must be 64 or 128 (others: SWA_ERR_UNSUPPORTED).
 *   - scale is the logit multiplier (1/sqrt(d_h) for the pages' attention);
 *     it must be finite and > 0.
 *   - Grouped-query heads: query head h reads key/value head h / (H_q / H_kv)
 *     (contiguous groups; H_q must be a multiple of H_kv).
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = default stream).
 *     Every argument is validated on the host before any HIP call; on error
 *     nothing is launched.  The library keeps no pointer after returning and
 *     allocates no device memory; its only global state is the per-GPU
 *     scratch array of swa_decode_noalloc and that array's cached address.
 *     Concurrent calls from several host threads are safe, except overlapping
 *     swa_decode_noalloc calls on one GPU (see there).
 *   - Errors: SWA_ERR_INVALID (bad argument), SWA_ERR_UNSUPPORTED (valid but
 *     not implemented), SWA_ERR_WORKSPACE (workspace too small), SWA_ERR_HIP
 *     (a HIP launch failed; device faults surface at stream synchronisation).
 *     The ABI never throws.
 */
#ifndef SWA_H
#define SWA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SWA_OK = 0,
  SWA_ERR_INVALID = 1,
  SWA_ERR_UNSUPPORTED = 2,
  SWA_ERR_WORKSPACE = 3,
  SWA_ERR_HIP = 4
} swa_status;

typedef enum { SWA_BF16 = 0, SWA_F32 = 1 } swa_dtype;

/* Window families for the introspection calls. */
enum { SWA_MODE_CAUSAL = 0, SWA_MODE_SYMMETRIC = 1 };

/* Causal sliding-window prefill.
 * Query t attends keys s with t-W < s <= t: W keys including itself, fewer at
 * the start (knowledge base §2: N_t = [max(0, t-W+1), t]; §3 mask; the Gemma 3
 * note's t=2000, W=1024 -> 977..2000).  W >= T is ordinary causal attention.
 *   q, o : [B, T, H_q, d_h]          k, v : [B, T, H_kv, d_h]
 *   lse  : [B, H_q, T] float32 natural-log sum of exp(logits), or NULL.
 * Errors: INVALID for null q/k/v/o, B,T,H_q,H_kv < 1, W < 1, H_q % H_kv != 0,
 * bad scale; UNSUPPORTED for other d_h. */
swa_status swa_prefill(swa_dtype dt, const void *q, const void *k, const void *v, void *o,
                       float *lse, int B, int T, int H_q, int H_kv, int d_h, int W,
                       float scale, void *stream);

/* Causal prefill with attention sinks.  Query t attends its window t-W < s <= t
 * united with the first n_sink positions s < n_sink, s <= t, each key once
 * (knowledge base §4 "Failure mode 1": StreamingLLM keeps the first few KV slots
 * pinned next to the rolling window; superteams.ai "What's New": sink positions
 * that every query sees).  sink_logit (device float32 [H_q], or NULL) gives each query
 * head a sink score z that joins the softmax denominator with no value:
 *   o = sum_s exp(e_s) v_s / (exp(z) + sum_s exp(e_s)),  lse = log(exp(z) + sum_s exp(e_s))
 * (a reading of the "learned per-head attention sink").  n_sink = 0 and a NULL
 * sink_logit is swa_prefill.  Arguments otherwise as swa_prefill.
 * Errors: as swa_prefill, plus INVALID for n_sink < 0, n_sink > 32 or a
 * misaligned sink_logit. */
swa_status swa_prefill_sinks(swa_dtype dt, const void *q, const void *k, const void *v, void *o,
                             float *lse, int B, int T, int H_q, int H_kv, int d_h, int W,
                             int n_sink, const float *sink_logit, float scale, void *stream);

/* Causal prefill with dilated windows.  Query t of head h attends the keys
 * t - i*d for 0 <= i < W that are >= 0, d = dilation[h] (knowledge base §2
 * "Dilation": the window {t - i*d : 0 <= i < W}, heads may use different d).
 * The key/value head of query head h is h / (H_q / H_kv) as in swa_prefill.
 *   dilation : HOST int32 [H_q], each in [1, 65535], or NULL (= all 1, which is
 *              swa_prefill); H_q <= 256 when some dilation is not 1
 * Arguments otherwise as swa_prefill.
 * Errors: as swa_prefill, plus INVALID for a dilation outside [1, 65535] and
 * UNSUPPORTED for more than 256 query heads with dilation. */
swa_status swa_prefill_dilated(swa_dtype dt, const void *q, const void *k, const void *v, void *o,
                               float *lse, int B, int T, int H_q, int H_kv, int d_h, int W,
                               const int32_t *dilation, float scale, void *stream);

/* Rotary position embedding, rotate-half form: for a token at position p the
 * pair (x_i, x_{i + d_h/2}) of every head turns by the angle p * base^(-2i/d_h):
 *   x_i' = x_i cos - x_{i+d/2} sin,   x_{i+d/2}' = x_{i+d/2} cos + x_i sin.
 * The Gemma 3 note ("How it works") keeps base 1e4 on local sliding-window
 * layers; the knowledge base (§2 "Interleaved local/global schemes") gives 1e4
 * local / 1e6 global.  The pairing is the common rotate-half convention.
 *   x, y : [B, T, H, d_h] device (y may equal x: in place)
 *   pos  : device int32 [B, T] positions, or NULL for p = t
 * Errors: INVALID for null or misaligned pointers, B, T, H < 1, a base that is
 * not finite and > 0; UNSUPPORTED for other d_h. */
swa_status swa_rope(swa_dtype dt, const void *x, void *y, const int32_t *pos, int B, int T, int H,
                    int d_h, float rope_base, void *stream);

/* Causal prefill with rotary positions applied to q and k first (positions
 * 0..T-1, base rope_base): the result is swa_prefill(rope(q), rope(k), v).
 * The queries are rotated in registers inside the prefill kernel; the keys are
 * rotated once into the workspace (every key feeds W / 32 query tiles, so
 * rotating inside the banded loop would repeat the work that often); q and k
 * are not modified.  The rotated values enter the MFMA products rounded to
 * bf16 (bf16 path).
 *   workspace : device scratch of at least swa_prefill_rope_workspace_size()
 *               bytes (the rotated keys, [B, T, H_kv, d_h]), 16-byte aligned.
 * Arguments otherwise as swa_prefill.  Errors: as swa_prefill, plus INVALID
 * for a bad base and WORKSPACE for a small workspace. */
size_t swa_prefill_rope_workspace_size(swa_dtype dt, int B, int T, int H_kv, int d_h);
swa_status swa_prefill_rope(swa_dtype dt, const void *q, const void *k, const void *v, void *o,
                            float *lse, int B, int T, int H_q, int H_kv, int d_h, int W,
                            float rope_base, float scale, void *workspace, size_t workspace_bytes,
                            void *stream);

/* Decode over a rolling-buffer KV cache: one new query token per request.
 * Token p is stored in slot p mod W (knowledge base §2 "KV cache"); every slot
 * records the absolute position it holds, and the window is computed from those
 * positions, not from slot offsets (Gemma 3 note, "How it works").  The caller
 * writes the current token into its slot first (swa_cache_write) and then calls
 * swa_decode.  Slot j is attended iff slot_pos[b][j] >= 0 and
 * cur_pos[b]-W < slot_pos[b][j] <= cur_pos[b]; slots holding stale or future
 * positions and empty slots (negative) are ignored, whatever bits their keys
 * and values hold (NaN or Inf included).  A request with no valid slot gets
 * o = 0 and lse = -inf.
 *   q, o             : [B, H_q, d_h]
 *   k_cache, v_cache : [B, H_kv, W, d_h]
 *   slot_pos         : [B, W] int32        cur_pos : [B] int32   (device)
 *   lse              : [B, H_q] float32 or NULL
 *   workspace        : device scratch of at least swa_decode_workspace_size()
 *                      bytes, 256-byte aligned, owned by the caller; contents
 *                      need not be initialised and are overwritten.
 * Errors: as swa_prefill, plus WORKSPACE when workspace_bytes is too small. */
size_t swa_decode_workspace_size(int B, int H_q, int H_kv, int W, int d_h);
swa_status swa_decode(swa_dtype dt, const void *q, const void *k_cache, const void *v_cache,
                      const int32_t *slot_pos, const int32_t *cur_pos, void *o, float *lse,
                      int B, int W, int H_q, int H_kv, int d_h, float scale, void *workspace,
                      size_t workspace_bytes, void *stream);

/* swa_decode without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  It allocates nothing: the split partial states go
 * to a scratch array of SWA_DECODE_NOALLOC_SCRATCH_BYTES that the library
 * holds in device memory, one per GPU, for the life of the process (its
 * address is looked up on the first call on a device; the calling thread's
 * current device is used, and `stream` must belong to it).  Every call on a
 * GPU shares that GPU's array and leaves its contents behind (nothing in it
 * needs to start at zero): calls that overlap on one GPU (other streams,
 * other threads) race on it; calls in one stream are ordered and safe.
 * Arguments, results and errors are those of swa_decode, plus
 * SWA_ERR_WORKSPACE when swa_decode_workspace_size() for the shape exceeds
 * SWA_DECODE_NOALLOC_SCRATCH_BYTES (nothing is launched then) and SWA_ERR_HIP
 * if the scratch address cannot be obtained. */
#define SWA_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
swa_status swa_decode_noalloc(swa_dtype dt, const void *q, const void *k_cache,
                              const void *v_cache, const int32_t *slot_pos,
                              const int32_t *cur_pos, void *o, float *lse, int B, int W, int H_q,
                              int H_kv, int d_h, float scale, void *stream);

/* Ring-cache append: writes k_new[b], v_new[b] ([B, H_kv, d_h]) into slot
 * pos[b] mod W of k_cache/v_cache ([B, H_kv, W, d_h]) and sets
 * slot_pos[b][slot] = pos[b] (knowledge base §2 "KV cache": writing token p
 * overwrites token p-W).  pos (device int32 [B]) must be >= 0. */
swa_status swa_cache_write(swa_dtype dt, const void *k_new, const void *v_new,
                           const int32_t *pos, void *k_cache, void *v_cache, int32_t *slot_pos,
                           int B, int W, int H_kv, int d_h, void *stream);

/* Ring-cache append of a chunk: token t of request b (k_new[b][t], v_new[b][t])
 * goes to slot pos[b][t] mod S, which records slot_pos[b][slot] = pos[b][t]
 * (knowledge base §2 "KV cache"; Gemma 3 note, "How it works").  The same rule
 * as swa_cache_write applied to each token; a ring of S >= W + L - 1 slots
 * keeps every key the chunk's own queries need after the append.  With n_sink
 * > 0 the first n_sink positions keep slots 0..n_sink-1 for good (pinned sink
 * tokens, knowledge base §4 "Failure mode 1") and later positions p roll over
 * the other slots: slot n_sink + (p - n_sink) mod (S - n_sink).
 *   k_new, v_new     : [B, L, H_kv, d_h]      pos : [B, L] int32 (device)
 *   k_cache, v_cache : [B, H_kv, S, d_h]      slot_pos : [B, S] int32
 * Preconditions (device data, not checked): pos >= 0 (negative tokens are
 * skipped) and the chunk's slots pos[b][t] mod S are distinct within each
 * request (true for consecutive positions with L <= S); otherwise which token
 * a shared slot keeps is unspecified.
 * Errors: INVALID for null pointers, B, L, S, H_kv < 1, L > S, B, L or H_kv >
 * 65535, n_sink < 0 or n_sink >= S; UNSUPPORTED for other d_h. */
swa_status swa_cache_append(swa_dtype dt, const void *k_new, const void *v_new,
                            const int32_t *pos, void *k_cache, void *v_cache, int32_t *slot_pos,
                            int B, int L, int S, int H_kv, int d_h, int n_sink, void *stream);

/* Chunked prefill over a ring cache (multi-token decode).  Query token t of
 * request b has absolute position q_pos[b][t] and attends the slots j with
 * slot_pos[b][j] >= 0 and q_pos[b][t]-W < slot_pos[b][j] <= q_pos[b][t]: the
 * window is computed from the positions stored with the cache (Gemma 3 note,
 * "How it works": M = 1[s > t-W] 1[s < t+W] with the causal s <= t), so slot
 * order, stale, future and empty slots do not matter.  Write the chunk's own
 * keys first (swa_cache_append) to let its queries see each other causally.
 * With n_sink > 0, slots holding one of the first n_sink positions (p <= q_pos)
 * are attended too; sink_logit as in swa_prefill_sinks (NULL = none).
 * A query with no valid slot gets o = 0 and lse = -inf (lse = z with a sink score).
 * Empty slots (negative position) may hold any bits (NaN or Inf included);
 * every other slot must hold finite keys and values, since a slot outside one
 * query's window may be inside another's of the same chunk.
 *   q, o             : [B, L, H_q, d_h]
 *   k_cache, v_cache : [B, H_kv, S, d_h]
 *   slot_pos         : [B, S] int32     q_pos : [B, L] int32, >= 0  (device)
 *   lse              : [B, H_q, L] float32 or NULL
 * No workspace.  Errors: INVALID for null pointers, B, L, S, H_q, H_kv < 1,
 * W < 1, H_q % H_kv != 0, bad scale, n_sink < 0, misaligned sink_logit;
 * UNSUPPORTED for other d_h or (bf16) a per-head cache slice of 2 GiB or more. */
swa_status swa_prefill_cached(swa_dtype dt, const void *q, const void *k_cache,
                              const void *v_cache, const int32_t *slot_pos, const int32_t *q_pos,
                              void *o, float *lse, int B, int L, int S, int H_q, int H_kv,
                              int d_h, int W, int n_sink, const float *sink_logit, float scale,
                              void *stream);

/* Longformer-style bidirectional attention.
 * A non-global row i of head h attends {i + k*dil[h] : -r <= k <= r} inside
 * [0, T) (prathamp.com §1.1 window, §3.1 dilation, §3.6 per-head dilation mix)
 * united with the global positions G_b, each counted once; a global row
 * (i in G_b) attends every position 0..T-1 (prathamp.com §4.3).
 *   q, k, v, o : [B, T, H, d_h]        lse : [B, H, T] float32 or NULL
 *   dilation   : HOST int32 [H], each in [1, 65535], or NULL (= all 1), H <= 256
 *   global_idx : HOST int32 [B, G]; each row strictly increasing in [0, T);
 *                NULL iff G == 0; B*G <= 512
 *   workspace  : device scratch of at least swa_longformer_workspace_size()
 *                bytes (0 when G == 0), 256-byte aligned, caller-owned.  With
 *                bf16 the global rows then come from partial states the banded
 *                pass leaves per 32-key block (B*H*G*n_blk records of d_h+4
 *                floats, n_blk = the most 32-key class blocks of any head; the
 *                reported size covers every head dilation up to 16); a head
 *                with a larger dilation, or a workspace too small for those
 *                records, takes a separate split-KV pass over K and V instead
 *                (same results within rounding).
 * Errors: INVALID for r < 0, bad dilation or global list, and the swa_prefill
 * cases; UNSUPPORTED for other d_h, H > 256 or B*G > 512; WORKSPACE. */
size_t swa_longformer_workspace_size(int B, int T, int H, int d_h, int G);
swa_status swa_longformer(swa_dtype dt, const void *q, const void *k, const void *v, void *o,
                          float *lse, int B, int T, int H, int d_h, int r,
                          const int32_t *dilation, const int32_t *global_idx, int G,
                          float scale, void *workspace, size_t workspace_bytes, void *stream);

/* Longformer-style attention with separate global projections (prathamp.com
 * §5.2: the global attention has its own query, key and value projections;
 * knowledge base §2 names Q_g, K_g, V_g).  The connectivity sets are those of
 * swa_longformer; what changes is which projection each pair reads:
 *   global row i (i in G_b): query qg_i against kg_s, vg_s for every s in [0, T);
 *   any other row i: query q_i against k_j, v_j for the window positions j
 *     that are not global, and against kg_g, vg_g for every global position g.
 * With qg, kg, vg equal to q, k, v this is swa_longformer (prathamp.com §5.3:
 * the global projections start as copies of the sliding ones).
 *   qg, kg, vg : [B, T, H, d_h] device, same dtype and layout as q, k, v
 *                (only the global rows of qg are read; kg, vg are read whole
 *                when G > 0)
 * Every other argument, the workspace size (swa_longformer_workspace_size)
 * and the errors are those of swa_longformer; null qg, kg or vg is INVALID. */
swa_status swa_longformer_proj(swa_dtype dt, const void *q, const void *k, const void *v,
                               const void *qg, const void *kg, const void *vg, void *o,
                               float *lse, int B, int T, int H, int d_h, int r,
                               const int32_t *dilation, const int32_t *global_idx, int G,
                               float scale, void *workspace, size_t workspace_bytes,
                               void *stream);

/* ---- introspection (tests)------------------------------------------------ */

/* Query/key tile sizes (rows per workgroup, keys per tile) the bf16 kernels use
 * for this entry point ('p' prefill, 'l' longformer) and head shape. */
swa_status swa_tile_config(int entry, int H_q, int H_kv, int d_h, int *BM, int *BN);

/* The band-tile schedule the kernels run (the same inline code): for each query
 * tile qi of BM rows and each key tile kj of BN columns it visits, one triple
 * (qi, kj, needs_mask) is written to out[3*n..3*n+2].  mode SWA_MODE_CAUSAL uses
 * window W = w_or_r; SWA_MODE_SYMMETRIC uses radius r = w_or_r (undilated: a
 * dilated head runs this schedule in each residue class, of length
 * ceil((T - rho) / dil)).  Returns the number of triples (which may exceed cap;
 * only the first cap are written), or -1 on invalid arguments.  Host only. */
int swa_band_tiles(int mode, int T, int w_or_r, int BM, int BN, int32_t *out, int cap);

/* Writes the connectivity sets as a uint8 [T, T] matrix (1 = attended) into
 * mask_dev (device), evaluated on the GPU from the per-row key bounds and the
 * residue-class mapping the banded kernels mask with (the same inline code).
 * It does not run the kernels' tile-level masking; that is read out through
 * the kernels themselves.  Causal: W = w_or_r.  Symmetric: r = w_or_r,
 * dilation dil, HOST global list global_idx[G]. */
swa_status swa_debug_index_mask(int mode, int T, int w_or_r, int dil, const int32_t *global_idx,
                                int G, uint8_t *mask_dev, void *stream);

const char *swa_status_str(swa_status s);
int swa_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SWA_H */
