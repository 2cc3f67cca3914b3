/*
 * sepattn.h -- C ABI of libsepattn: SepLLM separator-sparse attention and the
 * SepCache streaming decode on AMD Instinct MI355X (gfx950).
 *
 * What is computed (the pages' statement of the problem):
 *   * each query attends only to the first `a` initial tokens, every preceding
 *     separator token (a token whose id is in a fixed, hand-chosen set) and a
 *     local window of `n` neighbours (SepLLM summary on atlas.scime.ai,
 *     "Approach"; separator set: same page, "Limitations");
 *   * the output is attention restricted to that binary mask, O = M(A, V, M_b)
 *     ("How SepLLM Reorchestrates the Language Model for Speed and
 *     Efficiency", beiduofen.top, section "SepLLM's Architecture: Composing
 *     Efficiency"), read as softmax renormalised over the visible keys; the
 *     same mask is used in training (same page, "The Mechanics of
 *     Compression"), hence a forward and a backward;
 *   * streaming: a four-block KV cache (Initial, Local Window of capacity w,
 *     Past Window until usage reaches c, Separator Cache of capacity s) that is
 *     compressed when usage reaches c (beiduofen.top, "SepLLM's
 *     Architecture"; s on atlas.scime.ai, "Measured effects reported in the
 *     paper"), with positions re-assigned by cache slot (project card on
 *     sourcepulse.org, "Limitations & Caveats").
 *
 * Readings where the pages are silent: the window counts the query itself
 * (key j is in the window of query i iff i - j < n); grouped-query head h
 * reads kv head h / (Hq / Hkv); compression fires right after an append brings
 * usage to c and keeps the w newest window tokens; the Separator Cache keeps
 * its s newest entries; slot k of the cache (order Initial, Separator, Window)
 * has rotary position k; rotary embedding is the rotate-half form with
 * frequencies theta^(-2m/d).
 *
 * Conventions (every entry point):
 *   * Pointers are DEVICE pointers unless marked "host".  The caller owns all
 *     memory; the library never allocates or frees, keeps no global state
 *     (apart from the fixed decode scratch of sepcache_decode_noalloc) and
 *     may be called from several host threads on different streams.
 *   * `stream` is a hipStream_t passed as void*; all device work is enqueued
 *     on it and nothing synchronises the host.
 *   * Tensors are contiguous, innermost dimension last: Q/O/dO/dQ are
 *     [B, Hq, S, d], K/V/dK/dV are [B, Hkv, S, d], LSE is [B, Hq, S] fp32.
 *   * Every call returns a status code.  Argument errors are detected on the
 *     host before anything is enqueued; a kernel fault surfaces at the
 *     caller's next synchronisation of the stream.
 */
#ifndef SEPATTN_H
#define SEPATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define SEPATTN_OK 0
#define SEPATTN_EINVAL 1       /* null pointer, negative or zero size, a < 0, n < 1, Hq % Hkv != 0, scale <= 0, ... */
#define SEPATTN_EUNSUPPORTED 2 /* dtype / head-dim combination not built (d must be 64 or 128); one
                                  (sequence, head) slice S*d*element size at or above 2^31 bytes;
                                  more than 65535 query tiles of 128 rows, batch entries, or
                                  batch x kv-head pairs (launch grid dimensions); a SepCache with
                                  more than 128 kv heads (Hkv <= 128: one slot of every head, K and
                                  V, must fit the update kernel's 128 KB move chunk); a decode
                                  group Hq / Hkv that is not 1, 2, 4 or 8 */
#define SEPATTN_ECAPACITY 3    /* SepCache capacities: need w >= 1, s >= 0, a >= 0, c > a + s + w,
                                  and c <= 8192 (the update kernel plans a compression of the c
                                  slots in LDS) */
#define SEPATTN_EWORKSPACE 4   /* workspace smaller than the matching *_workspace() query */
#define SEPATTN_EHIP 5         /* a HIP launch failed */
#define SEPATTN_ESCRATCH 6     /* sepcache_decode_noalloc: the input needs more than the library's
                                  fixed scratch of SEPATTN_NOALLOC_SCRATCH_BYTES */

/* element types of Q/K/V/O and gradients */
#define SEPATTN_F32 0
#define SEPATTN_BF16 1

/* tile geometry of the index: 128 query rows x 64 keys */
#define SEPATTN_QTILE 128
#define SEPATTN_KTILE 64
/* number of int32 fields stored per query tile (6 defined, 2 reserved) */
#define SEPATTN_QTILE_FIELDS 8
/* largest separator id set accepted */
#define SEPATTN_MAX_SEP_IDS 64

/* Human-readable text of a status code (static storage). */
const char* sepattn_strerror(int status);

/* ------------------------------------------------------------------------ */
/* Index (separator positions and block-sparsity metadata)                   */
/* ------------------------------------------------------------------------ */

/*
 * Views into one caller-owned device buffer, carved by sepattn_index_bind.
 *   is_sep       [B, S]   uint8   1 iff the token id is in the separator set
 *   sep_prefix   [B, S+1] int32   sep_prefix[x] = number of separators at
 *                                 positions j with a <= j < x
 *   anchor_pos   [B, S]   int32   positions 0..min(a,S)-1, then every
 *                                 separator position >= a ascending, then -1
 *   anchor_count [B]      int32   min(a,S) + sep_prefix[S]
 *   qtile        [B, QT, 8] int32 for query tile qi (rows q0 = 128*qi ..
 *                                 q1 = min(q0+127, S-1)):
 *                                 [0] lo = max(0, q0 - n + 1)
 *                                 [1] n_anchor = anchors below lo
 *                                     = min(a, lo) + sep_prefix[lo]
 *                                 [2] kt_begin = lo / 64
 *                                 [3] kt_end = q1 / 64
 *                                 [4] n_kept = ceil(n_anchor/64) + kt_end - kt_begin + 1
 *                                 [5] rows = q1 - q0 + 1
 *                                 [6] q0
 *                                 [7] separators (at positions >= a) of the
 *                                     tile's two 64-position blocks: first
 *                                     block in bits 0..15, second in 16..31
 *   tile_class   [B, QT, KT] uint8 over the 128 x 64 grid of the S x S mask:
 *                                 0 no visible entry, 2 all visible, 1 otherwise
 * with QT = ceil(S/128), KT = ceil(S/64).  The visible keys of row i of tile
 * qi are exactly anchor_pos[0:n_anchor] (all < lo) plus the keys j in
 * [lo, i] that the mask keeps; the kernels visit ceil(n_anchor/64) gathered
 * anchor tiles and the key tiles kt_begin..kt_end.
 */
typedef struct {
  int B, S, a, n;
  uint8_t* is_sep;
  int32_t* sep_prefix;
  int32_t* anchor_pos;
  int32_t* anchor_count;
  int32_t* qtile;
  uint8_t* tile_class;
} sepattn_index;

/* Bytes of device memory an index for B sequences of length S needs. */
size_t sepattn_index_bytes(int B, int S);

/* Carve `buf` (device, >= sepattn_index_bytes(B,S) bytes, 256-byte aligned)
 * into the views of `idx` (host struct).  Nothing is enqueued.
 * EINVAL on null pointers or B, S < 1; EWORKSPACE if `bytes` is too small. */
int sepattn_index_bind(void* buf, size_t bytes, int B, int S, sepattn_index* idx);

/* Build the index of token ids `token_ids` [B, S] (device int32) for the
 * separator id set `sep_ids` (HOST array of n_sep int32, 0 <= n_sep <=
 * SEPATTN_MAX_SEP_IDS, read before the call returns), `a` initial tokens
 * (a >= 0) and window `n` (n >= 1).  idx must have been bound for the same
 * B and S; idx->a and idx->n are set, idx->n to min(n, S) (every n >= S
 * gives the same mask; sepattn_fwd and sepattn_bwd apply the same bound to
 * an idx->n set by hand).  Every output field is written.  One launch, two
 * from S >= 16384 on (a first one counts every tile's separators once, so
 * the work below each query tile reads counts instead of tokens); the
 * environment variable SEPATTN_INDEX_TWO_PASS_S, read at each call, moves
 * that length (0: never).  Both give the same output. */
int sepattn_build_index(const int32_t* token_ids, int B, int S, const int32_t* sep_ids, int n_sep,
                        int a, int n, sepattn_index* idx, void* stream);

/* Index of the fixed-interval baseline (FixLLM: anchors at fixed intervals
 * instead of separators; beiduofen.top, "Performance in the Spotlight:
 * Experimental Results"; atlas.scime.ai, "Surprising findings").  Position j
 * is an anchor iff j % interval == interval - 1 (interval >= 1), besides the
 * `a` initial tokens; no token ids are read.  Same outputs, binding rules and
 * errors as sepattn_build_index (EINVAL for interval < 1); sepattn_fwd and
 * sepattn_bwd take the result unchanged. */
int sepattn_build_index_interval(int B, int S, int interval, int a, int n, sepattn_index* idx, void* stream);

/* ------------------------------------------------------------------------ */
/* Attention over the full sequence (training / prefill)                     */
/* ------------------------------------------------------------------------ */

/* Forward.  q [B,Hq,S,d], k/v [B,Hkv,S,d] of `dtype`, scale > 0 (e.g. 1/sqrt(d)),
 * idx built for these B, S.  Writes o [B,Hq,S,d] (dtype) and lse [B,Hq,S]
 * fp32 = natural log of each row's softmax normaliser of the scaled scores.
 * Supported: dtype F32 or BF16 with d in {64, 128}.  Takes no workspace (and
 * so has no size query): every query tile's running statistics live in
 * registers and its K/V tiles in LDS. */
int sepattn_fwd(const void* q, const void* k, const void* v, int B, int Hq, int Hkv, int S, int d,
                int dtype, float scale, const sepattn_index* idx, void* o, float* lse, void* stream);

/* Device workspace bytes sepattn_bwd needs for these sizes. */
size_t sepattn_bwd_workspace(int B, int Hq, int Hkv, int S, int d, int dtype);

/* Backward of sepattn_fwd: given q, k, v, the forward's o and lse, and the
 * output gradient dout [B,Hq,S,d], writes dq [B,Hq,S,d], dk and dv
 * [B,Hkv,S,d] (dtype; dk/dv summed over the query heads of each group).
 * `ws` is device scratch of >= sepattn_bwd_workspace() bytes (256-byte
 * aligned); its contents on entry do not matter.  Supported: BF16 or F32,
 * d in {64, 128}. */
int sepattn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                const void* dout, int B, int Hq, int Hkv, int S, int d, int dtype, float scale,
                const sepattn_index* idx, void* dq, void* dk, void* dv, void* ws, size_t ws_bytes,
                void* stream);

/* sepattn_bwd with per-kernel timing: `events` is a HOST array of n_events
 * >= 4 hipEvent_t (created by the caller, passed as void*).  events[0] is
 * recorded on `stream` before the first kernel and events[i] after the i-th
 * of the three kernels: (1) query-major dQ, which also computes every row's
 * D = rowsum(dO * O) for the next kernel, (2) the main kernel (key-major
 * dK/dV over gathered anchor tiles and over band tiles, as one grid of
 * independent work items), (3) the sum of the anchor rows' partials, which
 * runs only when the anchor columns are split over several chunks of query
 * tiles (with one chunk the main kernel stores them and events[3] directly
 * follows events[2]).  A NULL entry records nothing at its point.  Results
 * are identical to sepattn_bwd. */
int sepattn_bwd_profiled(const void* q, const void* k, const void* v, const void* o, const float* lse,
                         const void* dout, int B, int Hq, int Hkv, int S, int d, int dtype, float scale,
                         const sepattn_index* idx, void* dq, void* dk, void* dv, void* ws, size_t ws_bytes,
                         void* stream, void* const* events, int n_events);

/* ------------------------------------------------------------------------ */
/* SepCache (streaming)                                                      */
/* ------------------------------------------------------------------------ */

/*
 * One cache per sequence of the batch, in caller-owned device buffers.
 * Slots [0, L) hold the Initial, Separator and Window blocks in that order,
 * L = n_init + n_sep + n_win <= c - 1 after every update.
 *   k, v   [B, Hkv, c, d] bf16 rows as appended (no rotary embedding)
 *   pos    [B, c] int32   stream position of the token in each slot, -1 if empty
 *   tok    [B, c] int32   token id of each slot, -1 if empty
 *   state  [B, 4] int32   n_init, n_sep, n_win, tokens seen
 * Requires Hkv >= 1, d in {64, 128}, a >= 0, s >= 0, w >= 1, c > a + s + w.
 */
typedef struct {
  int B, Hkv, d, c, a, s, w;
  void* k;
  void* v;
  int32_t* pos;
  int32_t* tok;
  int32_t* state;
} sepcache;

/* Empty every cache: counters 0, pos/tok -1 (k/v untouched). */
int sepcache_init(const sepcache* cache, void* stream);

/* Append one token per sequence: k_new/v_new [B, Hkv, d] bf16 (no rotary
 * embedding), tok_new [B] int32.  Takes no workspace (and so has no size
 * query): a compression's move plan lives in the LDS of one workgroup per
 * sequence.  The token joins the Initial block while it
 * holds fewer than a tokens, else the Window; if usage then equals c, the
 * Past Window (all but the w newest Window tokens) is compressed: its
 * separators (ids in `sep_ids`, HOST array of n_sep int32) join the Separator
 * block in stream order, the others are dropped, the Separator block keeps its
 * s newest entries and the cache is compacted.  Rows move bit for bit. */
int sepcache_update(const sepcache* cache, const void* k_new, const void* v_new,
                    const int32_t* tok_new, const int32_t* sep_ids, int n_sep, void* stream);

/* Prefill -> SepCache hand-off: sets every cache to what P calls of
 * sepcache_update with the prompt's tokens (after sepcache_init) would leave,
 * in one pass (the four blocks: beiduofen.top, "SepLLM's Architecture:
 * Composing Efficiency"; capacities: atlas.scime.ai, "Measured effects
 * reported in the paper").  k/v [B, Hkv, P, d] bf16 prompt rows (no rotary
 * embedding), tok [B, P] int32 device; idx = sepattn_build_index of tok with
 * the separator set the cache's later updates use and idx->a == cache->a (its
 * window n is not used).  Rows are copied bit for bit; pos/tok are written for
 * every slot and the counters set; earlier cache contents do not matter.
 * Work: one short recurrence per sequence (one step per compression until the
 * Separator block is full, then a closed form) and a copy of at most c - 1
 * rows.  EINVAL on null pointers, P < 1 or an index of another shape or `a`. */
int sepcache_prefill(const sepcache* cache, const void* k, const void* v, const int32_t* tok, int P,
                     const sepattn_index* idx, void* stream);

/* Device workspace bytes sepcache_decode needs for Hq query heads (the
 * size depends on Hq as well as on the cache: one fp32 partial per query
 * head and 128-slot chunk).  0 if the cache or Hq is invalid. */
size_t sepcache_decode_workspace(const sepcache* cache, int Hq);

/* Decode attention of the newest token of every sequence over its cache:
 * q [B, Hq, d] bf16 (no rotary embedding; Hq a multiple of Hkv with
 * Hq / Hkv in {1, 2, 4, 8}) is rotated at slot L-1, the key in slot k at
 * slot k, using rope_cos/rope_sin [c, d/2] fp32 (see
 * sepattn_rope_table_host); o [B, Hq, d] bf16 = softmax(scale q.K^T) V over
 * the L slots.  A sequence whose cache is empty (L = 0: nothing appended
 * since sepcache_init) gets o = 0.  `ws`: device scratch of >=
 * sepcache_decode_workspace() bytes, 256-byte aligned; its contents on entry
 * do not matter.  EWORKSPACE if ws_bytes is smaller. */
int sepcache_decode(const sepcache* cache, const void* q, int Hq, const float* rope_cos,
                    const float* rope_sin, float scale, void* o, void* ws, size_t ws_bytes,
                    void* stream);

/* Size of the device scratch the library keeps for sepcache_decode_noalloc
 * (per GPU, until the process ends). */
#define SEPATTN_NOALLOC_SCRATCH_BYTES (16u << 20)

/* sepcache_decode without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Same arguments (minus ws / ws_bytes),
 * results and errors as sepcache_decode, computed by the same kernels; the
 * chunk partials go to a fixed array of SEPATTN_NOALLOC_SCRATCH_BYTES in
 * device memory that the library holds on every GPU it runs on until the
 * process ends (its address is looked up on the first call on each device,
 * with `stream`'s device current).  Nothing is allocated or freed by the
 * call.  Limit: sepcache_decode_workspace(cache, Hq) must not exceed that
 * size (16 MiB: e.g. B = 64, Hq = 32, c = 800, d = 128 needs 7.5 MiB), else
 * ESCRATCH before any launch.  The array is shared by every call on one GPU
 * and keeps the last call's contents: calls that overlap on one GPU (on
 * different streams, or from several host threads) race and must be
 * serialised by the caller. */
int sepcache_decode_noalloc(const sepcache* cache, const void* q, int Hq, const float* rope_cos,
                            const float* rope_sin, float scale, void* o, void* stream);

/* sepcache_decode with per-kernel timing: `events` is a HOST array of
 * n_events >= 3 hipEvent_t (as void*), recorded on `stream` before the decode
 * kernel, after it, and after the kernel that merges its chunk partials.  A
 * NULL entry records nothing at its point.  Results are identical to
 * sepcache_decode. */
int sepcache_decode_profiled(const sepcache* cache, const void* q, int Hq, const float* rope_cos,
                             const float* rope_sin, float scale, void* o, void* ws, size_t ws_bytes,
                             void* stream, void* const* events, int n_events);

/* Host helper: cos/sin tables of the rotate-half rotary embedding,
 * cos_out[p*(d/2)+m] = cos(p * theta^(-2m/d)) (likewise sin), for p < c and
 * m < d/2, evaluated in double precision and rounded once to float.
 * cos_out/sin_out are HOST arrays of c*d/2 floats. */
int sepattn_rope_table_host(double theta, int c, int d, float* cos_out, float* sin_out);

#ifdef __cplusplus
}
#endif

#endif /* SEPATTN_H */
