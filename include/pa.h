/*
 * pa.h -- paged decode attention for AMD Instinct MI355X (gfx950), C ABI.
 *
 * The library implements the decode step over a paged KV cache:
 *   - pa_cache_append writes new K/V tokens into physical pages through a
 *     block table, quantising to FP8 e4m3 with per-(page, KV head) scales
 *     when the cache is FP8;
 *   - pa_decode checks the page tags a request expects, then runs grouped-
 *     query attention of one query token per sequence over every cached token;
 * and around it: pa_decode_step (a step's append and decode in one call),
 * pa_decode_multi (speculative verification of up to 8 draft tokens),
 * pa_prefill (chunked prefill), pa_decode_scored (eviction scores) and
 * pa_cache_compact (compaction after eviction).
 *
 * Sources (web pages; the citations name the page title and the passage):
 *   [paging]  "How we built the most efficient inference engine for
 *             Cloudflare's network", section "Batching to feed the Tensor
 *             Cores": the KV cache is split into pages assigned on demand, and
 *             each decoded token revisits all cached K/V of its sequence.
 *   [table]   "Making Workers AI faster and more efficient" (KV cache
 *             compression page), section "KV cache compression goes open
 *             source": a block table of integer indices maps a sequence onto
 *             blocks; a table per head lets heads keep different token counts.
 *   [fp8]     "Cloudflare quantizes Kimi and GLM caches for 41% faster
 *             inference", KV cache quantization paragraph: the cache is held
 *             in FP8 e4m3 instead of BF16, half the bytes, for the
 *             memory-bound decode phase.
 *   [tags]    same page, integrity-check paragraph: every physical page has a
 *             tag that changes on reallocation; the server records the
 *             (page, tag) pairs each request expects; a separate batch
 *             validation checks them before decode reads the cache; a request
 *             that fails is aborted; with checking off the tracker is a no-op.
 *   [evict]   "Making Workers AI faster and more efficient", section "KV cache
 *             compression goes open source": eviction drops the KV entries
 *             with the least accumulated past attention (a least-frequently-
 *             used policy); with a per-head block table every head can keep a
 *             different number of tokens.
 *
 * Conventions for every entry point:
 *   - All buffer pointers are DEVICE pointers unless stated otherwise; the
 *     descriptors themselves are host structs read during the call.
 *   - The caller owns every buffer.  The library allocates no device memory,
 *     keeps no state between calls, never synchronises the stream, and is
 *     reentrant.  Buffers must stay alive until the stream work completes.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream).
 *   - Argument errors return a negative PA_ERR_* code before anything is
 *     enqueued.  Data-dependent problems (bad page ids, stale tags, oversize
 *     lengths) are never returned: they set bits in the device `flags` array.
 *   - The element type of BF16 tensors is the raw 16-bit pattern (uint16_t).
 *
 * Physical cache layout (S = page_size = 16, D = head_dim in {64, 128},
 * e = bytes per element: 2 for BF16, 1 for FP8):
 *   SEQ  layout: K and V pools are [num_pages][num_kv_heads][block];
 *                block table int32 [batch][table_width]; lens int32 [batch].
 *   HEAD layout: K and V pools are [num_pages][block] (a page belongs to one
 *                (sequence, KV head) unit); table int32
 *                [batch][num_kv_heads][table_width]; lens [batch][num_kv_heads].
 *   A block holds the S x D elements of one (page, head).  Inside it the
 *   elements are arranged so that each 64-lane load of the decode kernel
 *   reads 1 KiB contiguously (let CE = 16 / e, elements per 16-byte chunk):
 *     K(t, d) at element  (d / (4*CE)) * (S * 4*CE) + t * (4*CE) + d % (4*CE)
 *             (the block is split into 64-byte column segments, each [S][4*CE]);
 *     V(t, d) with c = d % 16, j = d / 16, TPC = CE / 4 (tiles per chunk):
 *             at element ((((j / TPC) * 16 + c) * 4 + t / 4) * TPC + j % TPC) * 4 + t % 4
 *             (V is stored transposed, token-minor, in 16 x 4 MFMA tiles).
 *   The V block of logical (page p, head h) is stored in another pool slot
 *   than its K block, so that the two requests a decode wave makes for one
 *   page never meet at equal offsets of two alike-aligned pools (which costs
 *   HBM bank conflicts): SEQ with Hkv > 1 stores it in head (h + 1) % Hkv's
 *   slot of page p; otherwise in page (p ^ 1)'s slot, or p's own when p ^ 1
 *   is not below num_pages.
 *   Token t of a unit lives in page table[t / S], slot t % S.
 *   FP8 scales (float): SEQ [num_pages][num_kv_heads], HEAD [num_pages];
 *   the value of an element is decode_e4m3(code) * scale[page][head].
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *pa_stream_t; /* identical to hipStream_t */
typedef struct ihipEvent_t *pa_event_t;   /* identical to hipEvent_t */

enum { PA_LAYOUT_SEQ = 0, PA_LAYOUT_HEAD = 1 };
enum { PA_KV_BF16 = 0, PA_KV_FP8_E4M3 = 1 /* OCP E4M3 ("fn"): max 448, no inf */ };

enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = -1, /* null/misaligned pointer, bad size, bad enum */
  PA_ERR_UNSUPPORTED = -2, /* head_dim not 64/128, page_size not 16, GQA group > 16,
                              a page of all KV heads (Hkv x 16 x D x bytes) of 2^31 bytes or more */
  PA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than pa_decode_workspace_bytes */
  PA_ERR_LAUNCH = -4,      /* the HIP runtime refused a kernel launch */
  PA_ERR_SCRATCH = -5      /* pa_decode_noalloc: the call needs more than its static scratch */
};

/* Bits of the per-sequence flags word ([tags]: a request with any bit set is
 * to be aborted; its output rows are +0.0 and its pages are not read). */
enum {
  PA_FLAG_TAG_MISMATCH = 1u, /* expected tag != page tag for a page it would read */
  PA_FLAG_PAGE_OOB = 2u,     /* a page id it would read or write is outside [0, num_pages) */
  PA_FLAG_LEN_OVERFLOW = 4u, /* a length exceeds table_width * page_size */
  PA_FLAG_KEEP_INVALID = 8u  /* pa_cache_compact: a keep position outside [0, len) */
};

/* The physical cache ([paging], [table], [fp8], [tags]). */
typedef struct {
  int32_t layout;       /* PA_LAYOUT_SEQ or PA_LAYOUT_HEAD */
  int32_t kv_dtype;     /* PA_KV_BF16 or PA_KV_FP8_E4M3 */
  int32_t num_pages;    /* P */
  int32_t page_size;    /* S, must be 16 */
  int32_t num_kv_heads; /* Hkv */
  int32_t head_dim;     /* D, 64 or 128 */
  void *k_pages;        /* K pool, 256-byte aligned, layout above */
  void *v_pages;        /* V pool, 256-byte aligned, layout above */
  float *k_scale;       /* FP8 only (else NULL): per (page, head) */
  float *v_scale;       /* FP8 only (else NULL) */
  const uint32_t *page_tags; /* [P] current tag of every page; may be NULL when never validated */
} pa_cache_desc;

/* The logical view of one batch of sequences. */
typedef struct {
  int32_t batch;               /* B */
  int32_t table_width;         /* W, entries per table row */
  const int32_t *block_table;  /* SEQ [B][W], HEAD [B][Hkv][W]; entries past a unit's
                                  pages are never read */
  const int32_t *lens;         /* SEQ [B], HEAD [B][Hkv]: tokens held (decode: tokens attended) */
  const uint32_t *expected_tags; /* same shape as block_table; NULL = no-op tracker */
} pa_seq_desc;

/*
 * Size in bytes of one pool (K or V) for this cache shape: num_pages *
 * (Hkv for SEQ, 1 for HEAD) * S * D * e.  An FP8 pool is half a BF16 pool
 * ([fp8]).  Returns 0 for an invalid descriptor.
 */
size_t pa_pool_bytes(const pa_cache_desc *cache);

/*
 * Append tokens ([paging] pages assigned on demand, [fp8] quantisation).
 *
 * For every unit u (SEQ: sequence b, all heads; HEAD: (b, h)) writes the
 * n_new[u] tokens k_new/v_new[b][h][0 .. n_new[u]) at logical positions
 * seq->lens[u] .. seq->lens[u] + n_new[u] - 1 through the block table.
 *   n_new:  device int32, SEQ [B], HEAD [B][Hkv]; 0 <= n_new <= n_max.
 *   k_new, v_new: device BF16 [B][Hkv][n_max][D].
 *   seq->lens are the lengths BEFORE the append; the library never updates
 *   lengths or the table.
 *   seq->expected_tags (NULL or the table's shape; then cache->page_tags is
 *   required): a page is written only through a table entry whose expected
 *   tag equals the page's tag ([tags]: a stale entry may name a page that was
 *   reallocated to another request, whose tokens must not be overwritten).
 *   Tokens of a page that fails this test are not written.
 * BF16 caches get a copy of the bits.  FP8 caches, per (page, head) and
 * separately for K and V: s = fl32(amax / 448) over every value written since
 * the page was last started at slot 0 (a write starting at slot 0 resets the
 * page), codes = RNE_e4m3(saturate(fl32(x / s))); when the new values raise the
 * scale, codes already in the page are re-quantised as
 * RNE_e4m3(saturate(fl32(fl32(decode(c) * s_old) / s_new))).
 * Tokens whose page id is out of range, or beyond table_width * S, are not
 * written.  flags (device uint32 [B], may be NULL) is overwritten with
 * PA_FLAG_PAGE_OOB / PA_FLAG_LEN_OVERFLOW bits of this call, and with
 * PA_FLAG_TAG_MISMATCH for a page left alone because of its tag.
 * Pages must not be shared by two units within one call.
 */
int pa_cache_append(const pa_cache_desc *cache, const pa_seq_desc *seq, const int32_t *n_new,
                    int32_t n_max, const uint16_t *k_new, const uint16_t *v_new, uint32_t *flags,
                    pa_stream_t stream);

/*
 * Bytes of device workspace pa_decode needs for this shape and partition
 * count (0 = the library's choice).  0 when the decode needs none (one
 * partition per unit, SEQ layout).  Returns (size_t)-1 for invalid arguments.
 * The HEAD layout always adds one uint32 per unit (B * Hkv, rounded up to
 * 256 bytes) for the tag check, which validates each unit on its own.
 * With the automatic, length-balanced split (num_partitions 0, table_width
 * above 32) the size is the most any lengths can need: partials for
 * ceil(2048 / h) + groups (group, partition) pairs, where a group is a
 * sequence holding h = Hkv heads (SEQ) or one unit with h = 1 (HEAD), each
 * head G columns of D + 2 floats, plus the split plan: (groups + 3),
 * (pairs) and (4 * pairs) int32, every block rounded up to 256 bytes.
 */
size_t pa_decode_workspace_bytes(const pa_cache_desc *cache, const pa_seq_desc *seq,
                                 int32_t num_q_heads, int32_t num_partitions);

/* Number of token partitions pa_decode will use for this shape: the count
 * given, or for num_partitions == 0 the library's choice: 1 for tables of at
 * most 32 pages, else 0, which means balanced at run time (below).  Negative
 * PA_ERR_* on error. */
int pa_decode_num_partitions(const pa_cache_desc *cache, const pa_seq_desc *seq,
                             int32_t num_q_heads, int32_t num_partitions);

/*
 * Decode attention ([paging], [table], [fp8], [tags]).
 *
 * q: device BF16 [B][Hq][D], one query token per sequence; out: device BF16
 * [B][Hq][D].  Query head hq attends with KV head hq / (Hq / Hkv).  For each
 * unit, all lens[u] tokens are attended with scores softmax_scale * q.k,
 * softmax over tokens, output sum of weights * V, rounded to BF16 (nearest
 * even); fp32 accumulation.
 *
 * Integrity check: when seq->expected_tags != NULL, a separate validation
 * kernel runs first and overwrites flags[b] (required, device uint32 [B]) with
 * the PA_FLAG_* bits of sequence b over the ceil(len / S) entries each unit
 * reads.  When expected_tags == NULL but flags != NULL, only the page-range
 * and length bits are computed.  When both are NULL nothing is checked (the
 * no-op tracker): the caller guarantees valid ids and lengths; the kernels
 * still never read outside the pool or past table_width.
 * Rows of flagged sequences and of units with no tokens are written as +0.0.
 *
 * num_partitions: split of each unit's tokens (split-K) into that many
 * partitions of ceil(table_width / n) pages.  0 = automatic: for tables of
 * more than 32 pages the split is balanced on the device from the real
 * lengths -- one chunk size for the batch, about 2048 waves of equal work
 * (at least 32 pages each), so a ragged batch keeps every compute unit
 * streaming to the end.  The merge order then depends on the lengths; a
 * given input always gives the same bits.
 * workspace: device buffer of at least pa_decode_workspace_bytes(...) bytes,
 * 256-byte aligned (may be NULL when that size is 0).
 */
int pa_decode(const pa_cache_desc *cache, const pa_seq_desc *seq, int32_t num_q_heads,
              const uint16_t *q, uint16_t *out, float softmax_scale, int32_t num_partitions,
              uint32_t *flags, void *workspace, size_t workspace_bytes, pa_stream_t stream);

/*
 * pa_decode without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, serving loops and harnesses
 * that forbid hipMalloc.  Arguments, results, flags and error behaviour are
 * those of pa_decode, with the same kernels and the same split.
 *
 * The split-K partials and the split plan live in a static device array of
 * PA_NOALLOC_SCRATCH_BYTES (32 MiB), which every GPU the library runs on
 * holds until the process ends; its address is looked up once per device,
 * on that device's first call.  The call allocates nothing and issues no
 * memset: no scratch byte needs to start at zero, since every call writes
 * each byte it reads before reading it.
 *   - Every call on one GPU shares that GPU's array, which keeps the last
 *     call's contents: calls that overlap on one GPU (work on several
 *     streams, or from several host threads at once) race and give wrong
 *     results; calls ordered on one stream do not.
 *   - Make the call with the stream's device current (PA_ERR_INVALID_ARG
 *     otherwise).
 *   - A call that needs more than PA_NOALLOC_SCRATCH_BYTES (what
 *     pa_decode_workspace_bytes returns for the same arguments) returns
 *     PA_ERR_SCRATCH before anything is enqueued; pa_decode with a caller's
 *     workspace has no such limit.
 */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int pa_decode_noalloc(const pa_cache_desc *cache, const pa_seq_desc *seq, int32_t num_q_heads,
                      const uint16_t *q, uint16_t *out, float softmax_scale,
                      int32_t num_partitions, uint32_t *flags, pa_stream_t stream);

/*
 * pa_decode, plus timing events recorded on `stream` around its kernels:
 * events[0] before validation, events[1] before attention (after the split
 * plan, when automatic), events[2] after attention, events[3] after the
 * partition reduce.  Any entry may be NULL.
 */
int pa_decode_timed(const pa_cache_desc *cache, const pa_seq_desc *seq, int32_t num_q_heads,
                    const uint16_t *q, uint16_t *out, float softmax_scale, int32_t num_partitions,
                    uint32_t *flags, void *workspace, size_t workspace_bytes, pa_stream_t stream,
                    pa_event_t const events[4]);

/*
 * Multi-query decode: speculative verification of draft tokens.  The target
 * model checks every candidate token of a sequence in a single forward pass
 * ("Making Workers AI faster and more efficient", section "Speculative
 * decoding: predicting more than one token"; the extra-large-models write-up,
 * part 4, on draft-model speculative decoding).
 *
 * q: device BF16 [B][q_len][Hq][D]; out: device BF16 [B][q_len][Hq][D].
 * The q_len draft tokens are the LAST q_len tokens of every unit: the caller
 * appends them (pa_cache_append with n_new = q_len) before this call, and
 * seq->lens counts them.  Query token t (0-based) sits at position
 * lens[u] - q_len + t and attends tokens 0 .. lens[u] - q_len + t: the
 * earlier cache, the drafts before it, and itself (causal among the drafts).
 * A token with nothing to attend (lens[u] - q_len + t < 0) gets +0.0 rows.
 * Everything else -- scores, softmax, rounding, tag validation, flags,
 * partitions, workspace alignment -- is as pa_decode; q_len = 1 is pa_decode.
 *   q_len: 1 .. 8, and (Hq / Hkv) * q_len <= 64 when q_len > 1, else
 *          PA_ERR_UNSUPPORTED.
 * Workspace: pa_decode_multi_workspace_bytes(...) bytes (0 with one partition).
 */
int pa_decode_multi(const pa_cache_desc *cache, const pa_seq_desc *seq, int32_t num_q_heads,
                    int32_t q_len, const uint16_t *q, uint16_t *out, float softmax_scale,
                    int32_t num_partitions, uint32_t *flags, void *workspace,
                    size_t workspace_bytes, pa_stream_t stream);

/* pa_decode_multi with the four timing events of pa_decode_timed. */
int pa_decode_multi_timed(const pa_cache_desc *cache, const pa_seq_desc *seq,
                          int32_t num_q_heads, int32_t q_len, const uint16_t *q, uint16_t *out,
                          float softmax_scale, int32_t num_partitions, uint32_t *flags,
                          void *workspace, size_t workspace_bytes, pa_stream_t stream,
                          pa_event_t const events[4]);

/*
 * One decode step in one call: pa_cache_append of the step's new tokens,
 * then pa_decode (q_len = 1) or pa_decode_multi (q_len 2 .. 8) over them.
 * A decode step appends the token it produces before attending to it
 * (the caching of attention keys and values that the paging pages describe:
 * "How we built the most efficient inference engine for Cloudflare's
 * network", section "Batching to feed the Tensor Cores").
 *   seq:         the decode's view: seq->lens are the lengths after the
 *                append, and the appended tokens go through seq->block_table.
 *   lens_old:    device int32, seq->lens' shape: positions of the first new
 *                token; normally lens_old[u] + n_new[u] == seq->lens[u]
 *                (not checked).
 *   n_new, n_max, k_new, v_new: as pa_cache_append.
 *   everything else: as pa_decode / pa_decode_multi, including the workspace
 *   (their *_workspace_bytes) and the flags, which are the decode's
 *   validation of seq (the append itself sets no flag bits).  With
 *   seq->expected_tags the append writes only pages whose tag is the expected
 *   one, as pa_cache_append does; such a mismatch is also a mismatch of an
 *   entry the decode reads, so the sequence is flagged.
 * Pages, scales and outputs are bit-identical to the two calls made one after
 * the other.  The append shares the validation's launch (three launches
 * instead of four); errors as the two calls, checked before any launch.
 */
int pa_decode_step(const pa_cache_desc *cache, const pa_seq_desc *seq, const int32_t *lens_old,
                   const int32_t *n_new, int32_t n_max, const uint16_t *k_new,
                   const uint16_t *v_new, int32_t num_q_heads, int32_t q_len, const uint16_t *q,
                   uint16_t *out, float softmax_scale, int32_t num_partitions, uint32_t *flags,
                   void *workspace, size_t workspace_bytes, pa_stream_t stream);

/* pa_decode_step with the timing events of pa_decode_timed (events[0] is
 * recorded before the launch that appends and validates). */
int pa_decode_step_timed(const pa_cache_desc *cache, const pa_seq_desc *seq,
                         const int32_t *lens_old, const int32_t *n_new, int32_t n_max,
                         const uint16_t *k_new, const uint16_t *v_new, int32_t num_q_heads,
                         int32_t q_len, const uint16_t *q, uint16_t *out, float softmax_scale,
                         int32_t num_partitions, uint32_t *flags, void *workspace,
                         size_t workspace_bytes, pa_stream_t stream, pa_event_t const events[4]);

/*
 * Chunked prefill over the paged cache ([paging]: prefill processes the
 * prompt tokens in parallel; the batcher mixes decode with chunks of prefill
 * tokens -- "How we built the most efficient inference engine for
 * Cloudflare's network", section "Batching to feed the Tensor Cores").
 *
 * The same computation as pa_decode_multi with q_len = chunk_len, for chunks
 * of any length up to table_width * 16: the chunk's tokens are the last
 * chunk_len tokens of every unit (appended before the call); token t sees
 * tokens 0 .. lens[u] - chunk_len + t (the cached prefix and the chunk up to
 * itself).  q, out: device BF16 [B][chunk_len][Hq][D].
 * A unit's query columns (heads x chunk tokens) go to waves in blocks of 32,
 * four blocks per workgroup, whose waves share each page of the unit (staged
 * once through LDS; an FP8 page is also widened to bf16 / f16 operands there
 * once, each wave widening the quarter it loaded); a unit of at most 64
 * columns is one multi-query wave.
 * num_partitions (0 = automatic) splits the prefix only when the grid would
 * otherwise be small (the automatic choice aims at about 1536 workgroups).
 * Workspace: pa_prefill_workspace_bytes(...).
 */
int pa_prefill(const pa_cache_desc *cache, const pa_seq_desc *seq, int32_t num_q_heads,
               int32_t chunk_len, const uint16_t *q, uint16_t *out, float softmax_scale,
               int32_t num_partitions, uint32_t *flags, void *workspace, size_t workspace_bytes,
               pa_stream_t stream);

/* pa_prefill with the timing events of pa_decode_timed. */
int pa_prefill_timed(const pa_cache_desc *cache, const pa_seq_desc *seq, int32_t num_q_heads,
                     int32_t chunk_len, const uint16_t *q, uint16_t *out, float softmax_scale,
                     int32_t num_partitions, uint32_t *flags, void *workspace,
                     size_t workspace_bytes, pa_stream_t stream, pa_event_t const events[4]);

/* Workspace bytes of pa_prefill; (size_t)-1 for invalid arguments. */
size_t pa_prefill_workspace_bytes(const pa_cache_desc *cache, const pa_seq_desc *seq,
                                  int32_t num_q_heads, int32_t chunk_len, int32_t num_partitions);

/* Partitions pa_prefill will use (after the automatic choice when 0). */
int pa_prefill_num_partitions(const pa_cache_desc *cache, const pa_seq_desc *seq,
                              int32_t num_q_heads, int32_t chunk_len, int32_t num_partitions);

/* Workspace bytes of pa_decode_multi; (size_t)-1 for invalid or unsupported
 * arguments.  The partition count is pa_decode_num_partitions' (q_len does
 * not change it). */
size_t pa_decode_multi_workspace_bytes(const pa_cache_desc *cache, const pa_seq_desc *seq,
                                       int32_t num_q_heads, int32_t q_len,
                                       int32_t num_partitions);

/*
 * Decode that also updates eviction scores ([evict]).
 *
 * Everything pa_decode does and produces (q_len 1), bit for bit, plus: for
 * every unit that is not flagged, each of its lens[u] tokens gets the
 * softmax weight the step put on it, summed over the Hq / Hkv query heads of
 * the unit's KV head, added to its score:
 *   scores: device fp32, laid out like the pages -- SEQ [num_pages][Hkv][16],
 *           HEAD [num_pages][16]; entry (page, head, slot) is the token that
 *           K/V slot holds, so scores move with their pages.  Read and written
 *           in place (the caller zeroes a page's scores when it reallocates
 *           it).  Flagged sequences, slots past lens[u] and pages outside the
 *           pool (unchecked ids) are not touched.
 * The weights are those of the full softmax over the unit's tokens: after
 * the decode, a second pass reads the K pages again, recomputes the same fp32
 * scores the attention used (bitwise) and normalises them with the row's
 * final max and sum.  The sum over the query heads runs in a fixed order, so
 * repeated calls give the same bits.  num_partitions splits the decode
 * pass; the score pass splits the pages its own way.
 * Workspace: pa_decode_scored_workspace_bytes(...) bytes, never 0 (the
 * partials of pa_decode plus the rows' final max and sum, B * Hq * 8 bytes).
 * Data races: two concurrent calls on the same scores array race.
 */
int pa_decode_scored(const pa_cache_desc *cache, const pa_seq_desc *seq, int32_t num_q_heads,
                     const uint16_t *q, uint16_t *out, float softmax_scale,
                     int32_t num_partitions, uint32_t *flags, float *scores, void *workspace,
                     size_t workspace_bytes, pa_stream_t stream);

/* pa_decode_scored with the timing events of pa_decode_timed (events[3] is
 * recorded after the score update). */
int pa_decode_scored_timed(const pa_cache_desc *cache, const pa_seq_desc *seq,
                           int32_t num_q_heads, const uint16_t *q, uint16_t *out,
                           float softmax_scale, int32_t num_partitions, uint32_t *flags,
                           float *scores, void *workspace, size_t workspace_bytes,
                           pa_stream_t stream, pa_event_t const events[4]);

/* Workspace bytes of pa_decode_scored; (size_t)-1 for invalid arguments. */
size_t pa_decode_scored_workspace_bytes(const pa_cache_desc *cache, const pa_seq_desc *seq,
                                        int32_t num_q_heads, int32_t num_partitions);

/*
 * Compaction after eviction ([evict]): rewrite the tokens each unit keeps, in
 * the given order, from position 0 into the pages of a new table.
 *   seq:       the OLD table and lengths (seq->expected_tags is ignored).
 *   keep:      device int32 [B][Hkv][keep_stride]; keep[b][h][i] is the old
 *              position (0 <= p < lens) of the i-th token unit (b, h) keeps.
 *   n_keep:    device int32, lens' shape (SEQ [B]: every head of a sequence
 *              keeps the same number of tokens, as the SEQ layout has one
 *              length per sequence; HEAD [B][Hkv]: per head).  n_keep <=
 *              keep_stride and <= table_width * 16.
 *   new_table: device int32, the old table's shape; entries 0 ..
 *              ceil(n_keep / 16) - 1 of a row name the destination pages.
 *              They must not be pages this call reads (the caller allocates
 *              fresh pages and frees the old ones afterwards).
 *   scores:    NULL, or the eviction scores (see pa_decode_scored): each
 *              kept token's score moves with it.
 *   flags:     NULL or device uint32 [B], overwritten: PA_FLAG_PAGE_OOB for an
 *              old or new page id out of range, PA_FLAG_LEN_OVERFLOW for a
 *              length or count above the table or a count above keep_stride,
 *              PA_FLAG_KEEP_INVALID for a position outside [0, lens).  Such
 *              tokens are not written.
 * BF16 tokens are copied bit for bit.  FP8 tokens are decoded under their old
 * page scale, x = fl32(decode(c) * s_old), and re-quantised under the new
 * page's scale s = fl32(amax / 448) over the x the page receives, codes
 * RNE_e4m3(saturate(fl32(x / s))) -- the rule of an append into fresh pages.
 * Slots past n_keep in a unit's last new page are left as they were.  The
 * caller then uses new_table with lengths n_keep.
 */
int pa_cache_compact(const pa_cache_desc *cache, const pa_seq_desc *seq, const int32_t *keep,
                     int32_t keep_stride, const int32_t *n_keep, const int32_t *new_table,
                     float *scores, uint32_t *flags, pa_stream_t stream);

/* Static text for a PA_* return code. */
const char *pa_strerror(int code);

/* Library version, major * 10000 + minor * 100 + patch. */
int pa_version(void);

#ifdef __cplusplus
}
#endif
#endif /* PA_H_ */
