/*
 * swa.h — C ABI of libswa: causal sliding-window attention (SWA) and full attention over a
 * dual-pool KV cache, for AMD Instinct MI355X (gfx950).
 *
 * What the calls compute (sources are web pages, cited by title and section/equation):
 *
 *  [SWA-theory]  disassemble-channel.com, "Sliding Window Attention（SWA）の理論と実装 —
 *                固定窓による局所注意とMistralでの採用".
 *  [MiMo-review] youngju.dev review of Xiaomi's MiMo-V2.5 inference optimisation post.
 *
 *  - A query at absolute position i of a sequence sees the keys W(i) = {j : max(0,i-w+1) <= j <= i}
 *    in an SWA layer ([SWA-theory] §数学的定義 Eq.(1)) and all j <= i in a full layer.  Its output is
 *    softmax(q·k_j / sqrt(d)) over those keys applied to the values (Eq.(2)-(5); the scaled
 *    dot-product formula of §Full Attentionの問題点).  Query head h uses KV head h / (Hq/Hkv)
 *    (grouped-query attention, [SWA-theory] §MistralにおけるSWAの採用; contiguous groups).
 *  - Each SWA layer keeps a w-slot ring per sequence; position t lives in slot t mod w
 *    ([SWA-theory] §Rolling Buffer KV Cache, Eq.(7)).  Each full layer keeps every token in 16-token
 *    pages.  The two pools are separate ([MiMo-review] §潜在力を本番へ, dual-pool KV cache).
 *  - Reuse of a cached prefix is cut to the window-safe length ([MiMo-review] §潜在力を本番へ).
 *  - The hybrid stack marks some layers full (default: every 7th layer, l % 7 == 6, i.e. 10 of 70;
 *    [MiMo-review] §アーキテクチャ).
 *
 * Conventions for every call:
 *  - Return value 0 (SWA_OK) on success, a negative SWA_E* code otherwise; swa_last_error() then
 *    returns a thread-local message.  No C++ exception crosses this boundary.  On error no pool
 *    state has changed, unless the code is SWA_EHIP (a failed HIP call; the stream's work is then
 *    undefined).
 *  - Device pointers (q, k, v, out, workspace, the arena) are HIP device memory owned by the
 *    caller.  Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and is
 *    asynchronous: buffers must stay alive until the stream has passed the call.  The library keeps
 *    no pointer to q/k/v/out/workspace after a call returns.
 *  - Host pointers (desc, seqs, out-parameters) are read or written during the call only.
 *  - Tensors are dense row-major.  Prefill: q [n, Hq, d], k/v [n, Hkv, d], out [n, Hq, d].  Decode
 *    and verify: q [n_seqs, q_len, Hq, d], k_new/v_new [n_seqs, q_len, Hkv, d], out like q.  All of
 *    q, k, v and out are in the pool's dtype (fp32, or bf16 with fp32 accumulation inside).
 *  - A pool is not thread-safe.  All device work on one pool must go to one stream (or the caller
 *    orders streams itself): calls are ordered by the stream, host metadata by call order.
 *  - Attention is read-only on the pool: prior keys come from the pool, the new tokens' keys from
 *    the k/v arguments.  kvpool_append commits new tokens afterwards (e.g. only the accepted ones of
 *    a multi-token verify).  This order is required because a ring slot still holds a key that
 *    earlier queries of the same chunk need.
 */
#ifndef SWA_H
#define SWA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct swa_pool swa_pool; /* opaque; host metadata owned by the library */

/* SWA_F32 and SWA_BF16 pools store and compute in that dtype.  SWA_FP8_E4M3 is a storage dtype
 * only ([MiMo-review] §おわりに: the window-limited cache can itself be stored in FP8): K/V entries
 * are kept as OCP E4M3 codes (1 byte) with a per-pool power-of-two scale (see swa_pool_desc);
 * appends take bf16 K/V and quantise them, attention calls take bf16 activations and read
 * dequantised keys and values. */
typedef enum { SWA_F32 = 0, SWA_BF16 = 1, SWA_FP8_E4M3 = 2 } swa_dtype;

/* Coordinate pairs that RoPE rotates together (see kvpool_rope): (2i, 2i+1), the RoFormer paper's
 * layout, or (i, i + d/2), the split-halves layout of GPT-NeoX-style models. */
typedef enum { SWA_ROPE_PAIRS = 0, SWA_ROPE_HALVES = 1 } swa_rope_style;

/* Work planner of full-layer decode / verify calls (which keys each split-K work item reads).
 * SWA_PLAN_UNIFORM: one split size for the whole call, chosen so the items fill whole rounds of
 * the GPU; items in sequence order.  SWA_PLAN_BUCKETED: sequences grouped by prior length into the
 * buckets 0-64K, 64K-256K and 256K and more ([MiMo-review] §潜在力を本番へ: length bucketing keeps
 * batches homogeneous); each bucket gets its own round-filling split, and the work list runs the
 * longest bucket first, whole splits before the shorter tail pieces.  Results are the same up to
 * floating-point summation order. */
typedef enum { SWA_PLAN_UNIFORM = 0, SWA_PLAN_BUCKETED = 1 } swa_decode_plan;

enum {
  SWA_OK = 0,
  SWA_EINVAL = -1, /* invalid argument, shape, dtype, or call not allowed in this state */
  SWA_ENOSEQ = -2, /* sequence id out of range, or not open */
  SWA_ENOMEM = -3, /* out of pages or sequence slots; arena or workspace too small */
  SWA_EHIP = -4    /* a HIP runtime call or kernel launch failed (see swa_last_error) */
};

typedef struct {
  int32_t n_layers;              /* >= 1 */
  const uint8_t *layer_is_full;  /* n_layers flags (nonzero = full attention layer), copied at
                                    create; NULL = default hybrid map (l % 7 == 6 is full) */
  int32_t window;                /* w >= 1: ring slots per SWA layer and the attention window */
  int32_t n_kv_heads;            /* Hkv >= 1 */
  int32_t head_dim;              /* d: 64 or 128 */
  swa_dtype kv_dtype;            /* storage dtype of the whole pool (compute: see swa_dtype) */
  int32_t page_tokens;           /* tokens per full-layer page; must be 16 */
  int64_t pages_per_full_layer;  /* page capacity of each full layer (>= 0) */
  int32_t max_seqs;              /* sequence slots (>= 1) */
  int64_t max_seq_len;           /* longest sequence the page tables can map, 1 .. 2^31 - 1
                                    (key indices inside the kernels are 32-bit) */
  int32_t max_snapshots;         /* ring snapshots the arena holds (>= 0), see kvpool_snapshot */
  float k_scale, v_scale;        /* SWA_FP8_E4M3 pools: positive powers of two in [2^-60, 2^60]
                                    (0 means 1).  A value x is stored as the E4M3 code nearest to
                                    x / scale (ties to even, saturating at +-448) and a code c reads
                                    as e4m3(c) * scale, exactly.  Ignored for other dtypes. */
  float rope_base;               /* RoPE frequency base (e.g. 10000), or 0: the pool has no RoPE
                                    tables and kvpool_rope is SWA_EINVAL.  With RoPE the arena also
                                    holds angle tables of (2048 + ceil(max_seq_len / 2048)) * d * 4
                                    bytes (built on the host at create), and max_seq_len must
                                    be <= 2^26. */
  int32_t rope_style;            /* swa_rope_style (checked even without RoPE) */
  int32_t decode_plan;           /* swa_decode_plan */
  int32_t rope_fused;            /* 1: RoPE inside the attention and commit calls (see below);
                                    needs rope_base > 0, a bf16 or FP8 pool and max_chunk >= 1 */
  int32_t max_chunk;             /* rope_fused pools: the longest prefill chunk (tokens); the arena
                                    holds the chunk's rotated keys, max_chunk * Hkv * d * 2 bytes */
} swa_pool_desc;

/* ---------------------------------------------------------------------------------------------
 * Pool lifetime.  The arena is one device allocation made by the caller, of
 * kvpool_arena_bytes(desc) bytes (256-byte aligned).  It holds the SWA rings (w slots per
 * sequence, layer and KV head: O(W)), the full-layer pages (O(N)) and the device copies of the
 * page tables.  It must outlive the pool.
 * ------------------------------------------------------------------------------------------- */

/* Arena size for `d`, or a negative SWA_E* code if `d` is invalid. */
int64_t kvpool_arena_bytes(const swa_pool_desc *d);

/* Create a pool over `dev_arena` (arena_bytes >= kvpool_arena_bytes(d)).  dev_arena == NULL
 * creates a planning pool: host metadata only (sequences, lengths, pages, ring tags, bytes,
 * window-safe length, fork and append bookkeeping with k/v ignored); attention calls on it return
 * SWA_EINVAL.  Pinned host staging memory (a few MiB) is allocated for arena-backed pools. */
int kvpool_create(const swa_pool_desc *d, void *dev_arena, int64_t arena_bytes, swa_pool **out);

/* Free host metadata and staging memory; waits for the pool's pending staging copies.  The
 * arena is not touched.  NULL is accepted. */
int kvpool_destroy(swa_pool *p);

/* Open an empty sequence (length 0 in every layer); *seq receives its id in [0, max_seqs). */
int kvpool_seq_open(swa_pool *p, int32_t *seq);

/* Close a sequence: drop one reference to each of its pages (a page returns to its layer's free
 * list at zero) and free its ring slots.  Work already enqueued that reads it must be ordered
 * before any later call that reuses the slot or the pages (same stream). */
int kvpool_seq_close(swa_pool *p, int32_t seq);

/* ---------------------------------------------------------------------------------------------
 * Prefix reuse ([MiMo-review] §潜在力を本番へ: SWA-aware prefix cache, window-safe length).
 * ------------------------------------------------------------------------------------------- */

/* Largest m' <= min(match_len, committed length of `donor`) such that in every SWA layer of the
 * donor each position p in [max(0, m'-w), m') still sits in its ring slot (slot p mod w holds p).
 * The page's "last W tokens" is read literally (w positions).  m' = 0 always qualifies.  With
 * contiguous appends this is m if the donor never exceeded w tokens or m equals its length, else
 * 0.  Host only; touches no device memory.  match_len < 0 is SWA_EINVAL. */
int kvpool_window_safe_len(const swa_pool *p, int32_t donor, int64_t match_len, int64_t *out);

/* Open a new sequence whose first `reuse_len` tokens, in every layer, are the donor's.
 * reuse_len must be window-safe (kvpool_window_safe_len(donor, reuse_len) == reuse_len), else
 * SWA_EINVAL: reusing ring contents past that point would silently read other positions.
 * Full layers share the donor's whole pages below reuse_len by reference (refcount) and copy the
 * partial last page into a new page; SWA layers copy the donor's ring.  Copies are enqueued on
 * `stream`.  SWA_ENOMEM if no sequence slot or page is free. */
int kvpool_seq_fork(swa_pool *p, int32_t donor, int64_t reuse_len, int32_t *seq, void *stream);

/* Window snapshots for a prefix-cache tree.  A plain ring only supports reuse up to the window
 * (or of a donor's whole history): once a donor grows past m + w, the ring no longer holds the w
 * tokens before m.  A snapshot keeps them: it copies the sequence's SWA rings (all SWA layers, at
 * its committed length m, which must be the same in every layer) into one of the arena's
 * max_snapshots slots and holds a reference on the full-layer pages covering [0, m), so the
 * donor may grow, fork or close afterwards.  *snap receives the slot id.  SWA_ENOMEM if no slot is
 * free.  The copy is enqueued on `stream`. */
int kvpool_snapshot(swa_pool *p, int32_t seq, int32_t *snap, void *stream);

/* Open a new sequence whose first m tokens (m = the snapshot's length), in every layer, are the
 * snapshotted ones: SWA rings restored from the snapshot, whole full-layer pages below m shared by
 * reference, the partial last page copied into a new page.  SWA_ENOMEM if no sequence slot or page
 * is free.  Copies are enqueued on `stream`. */
int kvpool_seq_fork_snapshot(swa_pool *p, int32_t snap, int32_t *seq, void *stream);

/* Length m of a snapshot. */
int kvpool_snapshot_len(const swa_pool *p, int32_t snap, int64_t *len);

/* Drop a snapshot: its page references (a page returns to its free list at zero) and its slot.
 * Work already enqueued that reads it must be ordered before any later snapshot into the slot. */
int kvpool_snapshot_release(swa_pool *p, int32_t snap);

/* ---------------------------------------------------------------------------------------------
 * Commit ([SWA-theory] §Rolling Buffer KV Cache Eq.(7); full layers: paged O(N) pool).
 * ------------------------------------------------------------------------------------------- */

/* Append n >= 1 tokens (k, v: [n, Hkv, d] device; fp32 for SWA_F32 pools, bf16 for SWA_BF16 and
 * SWA_FP8_E4M3 pools, which quantise them as swa_pool_desc states) at positions L .. L+n-1 of
 * (seq, layer), L = kvpool_seq_len.  SWA layer: position p goes to ring slot p mod w; only the
 * last min(n, w) tokens are written (earlier ones would be overwritten within the same call).
 * Full layer: pages for the new positions are taken from the layer's free list (SWA_ENOMEM with
 * no change if too few) and position p goes to page table[p / 16], row p % 16.  K and V are
 * stored as [Hkv][tokens][d] per ring (tokens = w slots) or page (16 rows). */
int kvpool_append(swa_pool *p, int32_t seq, int32_t layer, const void *k, const void *v, int32_t n,
                  void *stream);

/* Commit n >= 1 new tokens to each of n_seqs >= 1 distinct sequences in one launch (a decode
 * step's commit): k, v are [n_seqs, n, Hkv, d]; sequence seqs[i] takes rows [i*n, (i+1)*n) at its
 * positions L_i .. L_i+n-1.  Placement, dtype and atomicity (no change on SWA_EINVAL/SWA_ENOMEM)
 * as kvpool_append.  Page-table updates and the sequence list travel through a 4 MiB landing zone
 * at the end of the arena, in stream order. */
int kvpool_append_batch(swa_pool *p, int32_t n_seqs, const int32_t *seqs, int32_t layer, const void *k,
                        const void *v, int32_t n, void *stream);

/* ---------------------------------------------------------------------------------------------
 * RoPE.  [SWA-theory] §Rolling Buffer KV Cache: ring slots hold keys out of time order, which is
 * harmless because rotary position embedding writes each token's absolute position into its query
 * and key, so scores depend on positions, not slots.  The rotation is RoFormer's (Su et al., 2021,
 * §3.2-§3.4): pair i of a head vector (desc.rope_style) turns by p * theta_i at position p,
 * theta_i = rope_base^(-2i/d), counter-clockwise (x + iy times e^(i p theta_i)).
 * ------------------------------------------------------------------------------------------- */

/* Fused RoPE (swa_pool_desc.rope_fused = 1).  Attention calls (swa_attn_prefill,
 * swa_attn_decode, full_attn, full_attn_noalloc) then take q and the call's keys unrotated:
 * every query row is rotated at its position inside the attention kernel as it is loaded; the
 * call's new keys are rotated at their positions as the decode kernel loads them, and a prefill
 * call first writes its chunk's rotated keys into the arena (one pass over the keys only), where
 * the attention kernel reads them.  Commits (kvpool_append, kvpool_append_batch) take the keys
 * unrotated as well and rotate them as they store them, so the pool holds rotated keys as with
 * kvpool_rope.  Values are never rotated; the caller's q, k and v are never written.  Results
 * equal those of kvpool_rope followed by the unfused calls (same rotation arithmetic, one bf16
 * rounding).  kvpool_rope stays available on such pools for callers that need rotated vectors
 * themselves (passing its output to a fused call would rotate twice).  The chunk's rotated keys
 * share one arena region per pool: prefill calls on one fused pool issued on different streams
 * must not overlap in time. */

/* Rotate, in place and in one launch, the queries q [n_seqs, n, n_q_heads, d] and the keys
 * k [n_seqs, n, Hkv, d] (activation dtype dt, as for attention) of n_seqs >= 1 sequences at the
 * positions the next attention call gives them: token t of seqs[i] at L_i + t, L_i = committed
 * length of (seqs[i], layer).  Either q or k may be NULL (then n_q_heads is ignored for q).  Call it
 * before attention; the rotated keys are the ones to pass to attention and then to kvpool_append
 * (the pool stores rotated keys; values are never rotated).  Angles come from float64 tables in the
 * arena, so positions up to max_seq_len keep fp32 accuracy; results are rounded to dt (bf16: nearest
 * even).  SWA_EINVAL for a pool without RoPE, a planning pool, L_i + n > max_seq_len, or a dtype
 * mismatch.  Several sequences: their first positions travel through the arena's landing zone, in
 * stream order. */
int kvpool_rope(swa_pool *p, int32_t n_seqs, const int32_t *seqs, int32_t layer, void *q, int32_t n_q_heads,
                void *k, int32_t n, swa_dtype dt, void *stream);

/* Committed length of (seq, layer). */
int kvpool_seq_len(const swa_pool *p, int32_t seq, int32_t layer, int64_t *len);

/* KV bytes of the open sequences: the pool-level form of the KV-size calculator of [SWA-theory]
 * §計算時間・メモリ比較実験 (2 x tokens x Hkv x d x element bytes per layer, with an SWA layer
 * holding at most w tokens), summed over the hybrid stack whose total [MiMo-review] §アーキテクチャ
 * puts at (60 W + 10 N) / (70 N) of an all-full cache.  allocated: w slots per SWA layer and 16 rows
 * per full-layer page held; resident: min(L, w) live slots per SWA layer plus the pages.  A page
 * shared by several sequences counts once.  Either pointer may be NULL. */
int kvpool_bytes(const swa_pool *p, int64_t *allocated, int64_t *resident);

/* Layer kind of `layer`: 1 full attention, 0 SWA; negative on error. */
int kvpool_layer_is_full(const swa_pool *p, int32_t layer);

/* Free pages of a full layer. */
int kvpool_free_pages(const swa_pool *p, int32_t layer, int64_t *n_free);

/* Where position `pos` of (seq, layer) lives for KV head `head`, as byte offsets into the arena:
 * the key row at *k_off and the value row at *v_off, each d elements with *v_stride bytes between
 * consecutive dims (the element size).  SWA_EINVAL if the position is not resident (beyond the
 * length, or overwritten in the ring).  For tests and tools. */
int kvpool_locate(const swa_pool *p, int32_t seq, int32_t layer, int64_t pos, int32_t head,
                  int64_t *k_off, int64_t *v_off, int64_t *v_stride);

/* Ring tags of (seq, SWA layer): tags[s] = the position slot s holds, or -1.  `tags` has w
 * entries. */
int kvpool_slot_tags(const swa_pool *p, int32_t seq, int32_t layer, int64_t *tags);

/* ---------------------------------------------------------------------------------------------
 * Attention.  dt is the activation dtype: SWA_F32 for SWA_F32 pools, SWA_BF16 for SWA_BF16 and
 * SWA_FP8_E4M3 pools; n_q_heads must be a multiple of Hkv.  Keys and values already in an FP8
 * pool are read dequantised (e4m3(c) * scale); the call's own new tokens are used as passed.
 * ------------------------------------------------------------------------------------------- */

/* SWA prefill of one chunk ([SWA-theory] Eq.(1)-(5); chunked prefill with the prefix carried in
 * the ring: §発展的な話題, and [MiMo-review] §潜在力を本番へ, 16K chunks).  Queries at positions
 * L .. L+n-1 of (seq, layer), L = committed length, n >= 1 (any chunk size; at most max_chunk on a
 * rope_fused pool).  Keys j < L come from
 * the ring (they are all still resident: i-w+1 >= L-w+1), keys j >= L from k/v.  Whole key tiles
 * outside the band are skipped.  Does not append. */
int swa_attn_prefill(swa_pool *p, int32_t seq, int32_t layer, const void *q, const void *k,
                     const void *v, int32_t n, int32_t n_q_heads, swa_dtype dt, void *out,
                     void *stream);

/* SWA decode / multi-token verify for n_seqs >= 1 sequences (distinct ids), q_len in 1..4: the
 * queries of sequence s sit at positions L_s .. L_s+q_len-1, the new keys/values in k_new/v_new.
 * Each row attends over W(i) of [SWA-theory] Eq.(1)-(5), reading the prior keys from the rolling
 * buffer in slot order (§Rolling Buffer KV Cache: generation reads the w-slot cache one token at a
 * time; slot order is harmless under RoPE); q_len up to 4 is the one-pass check of the 3 draft
 * tokens of multi-token prediction ([MiMo-review] §アーキテクチャ).  The one stale slot
 * (position L_s - w) is masked by position.  workspace: device memory of
 * >= swa_attn_workspace_bytes(...) bytes, 256-byte aligned (SWA_ENOMEM if smaller). */
int swa_attn_decode(swa_pool *p, int32_t n_seqs, const int32_t *seqs, int32_t layer,
                    const void *q, const void *k_new, const void *v_new, int32_t q_len,
                    int32_t n_q_heads, swa_dtype dt, void *out, void *workspace, int64_t ws_bytes,
                    void *stream);

/* Full attention over the paged pool: the full-attention layers of the hybrid stack, whose KV
 * grows as O(N) in a pool of their own ([MiMo-review] §アーキテクチャ and §潜在力を本番へ, dual-pool
 * KV cache; the scaled dot-product softmax of [SWA-theory] §Full Attentionの問題点 over every
 * j <= i).  q_len_or_chunk <= 4: decode / verify for n_seqs sequences (as swa_attn_decode, over all
 * prior tokens, split over pages with a log-sum-exp merge).  q_len_or_chunk > 4: prefill of one
 * chunk (n_seqs must be 1; tensors as for swa_attn_prefill; the 16K chunks of [MiMo-review]
 * §潜在力を本番へ): queries at L .. L+n-1 see all prior pages and the chunk causally.
 * workspace: >= swa_attn_workspace_bytes(...) bytes, 256-byte aligned (may be NULL with ws_bytes 0
 * for prefill). */
int full_attn(swa_pool *p, int32_t n_seqs, const int32_t *seqs, int32_t layer, const void *q,
              const void *k_new, const void *v_new, int32_t q_len_or_chunk, int32_t n_q_heads,
              swa_dtype dt, void *out, void *workspace, int64_t ws_bytes, void *stream);

/* full_attn for callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the same computation, arguments and errors as
 * full_attn without the workspace, which instead is a 32 MiB device array inside the library, one
 * per GPU, held until the process ends.  Calls whose swa_attn_workspace_bytes exceeds 32 MiB
 * return SWA_ENOMEM (e.g. a decode step whose split-K partials exceed it; use full_attn with a
 * workspace then).  The call allocates nothing (no hipMalloc, no library allocation).  Every call
 * on one GPU uses that GPU's array, which keeps the last call's contents (nothing in it needs to
 * start at zero): calls that overlap on one GPU (other streams, other threads) race on it. */
int full_attn_noalloc(swa_pool *p, int32_t n_seqs, const int32_t *seqs, int32_t layer, const void *q,
                      const void *k_new, const void *v_new, int32_t q_len_or_chunk, int32_t n_q_heads,
                      swa_dtype dt, void *out, void *stream);

/* Workspace bytes swa_attn_decode / full_attn need for this call (0 for a full-layer prefill).
 * Negative SWA_E* on invalid arguments. */
int64_t swa_attn_workspace_bytes(const swa_pool *p, int32_t n_seqs, const int32_t *seqs,
                                 int32_t layer, int32_t q_len_or_chunk, int32_t n_q_heads);

/* Message of the last failed call on this thread ("" if none). */
const char *swa_last_error(void);

/* Measurement aid, not a step of the method: enqueues on `stream` one lane that reads the GPU's
 * shader-clock counter and its fixed-rate wall clock, sleeps until spin_us microseconds of wall
 * time have passed, and reads both again.  Run on a second stream beside a timed kernel, it gives
 * the shader clock the device ran at meanwhile: (out[1]-out[0]) / (out[3]-out[2]) * out[4] kHz.
 * out: device memory, 5 int64, 8-byte aligned, written when the lane finishes (shader clock at
 * start, at end; wall clock at start, at end; wall clock rate in kHz).  spin_us in 1 .. 10^7.
 * SWA_EINVAL on a NULL or misaligned out or spin_us out of range, SWA_EHIP if the launch fails. */
int swa_clock_probe(void *out, int64_t spin_us, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SWA_H */
