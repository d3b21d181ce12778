/*
 * segpaged.h -- SegPagedAttention for AMD Instinct MI355X (gfx950).
 *
 * A KV cache paged per (layer, KV head, segment) and mask-free attention that
 * reads each head's own page list and length.
 *
 * Sources (the method this library implements):
 *   [RT]  "How different attention heads see different contexts: RedKnot
 *         SegPagedAttention paged-attention runtime design" (m.nxbn.cn/news/186605)
 *         -- section 2: the four per-(layer, KV head) policies; section 3: the
 *         (layer, head, segment) -> contiguous virtual pages table, the page
 *         pool, building per-head storage from dense KV; section 4: the
 *         mask-free fused varlen kernel and the dense+mask equivalence check;
 *         section 5: layout must be built once at KV-write time.
 *   [SUM] RedKnot summary (m.youleyou.com/wenzhang/3087667.html) -- head-class
 *         sparsification; SegPagedAttention as storage + execution substrate;
 *         system gains (KV bytes moved between prefill and decode machines).
 *   [KV]  KV-cache guide (zhangjiuzhi.com/?p=3078) -- section 4.3 block tables,
 *         section 5.3 GQA grouping, section 10.2 online softmax.
 *
 * Conventions for every call:
 *   - All functions are C, never throw, and return a segpaged_status (0 = OK,
 *     negative = error). Arguments are validated before any GPU work is enqueued;
 *     on error nothing is enqueued and outputs are untouched.
 *   - The library never allocates or frees device memory and never synchronises
 *     a stream. Device buffers (pools, table, Q, O, LSE, workspace, dense K/V)
 *     are owned by the caller. `stream` is a hipStream_t passed as void*
 *     (NULL = the null stream) on the current HIP device.
 *   - k_pool and v_pool may be NULL when the plan has no pages (pool_bytes = 0:
 *     no head keeps a token), and a page stream of zero elements may be NULL.
 *   - Asynchronous kernel faults surface at the caller's next synchronisation.
 *   - bf16 tensors are raw IEEE bfloat16 bits, row-major, 16-byte aligned.
 *   - A plan's layout changes only in segpaged_plan_append (growth plans); every
 *     other call reads it (segpaged_prefill also advances an atomic launch
 *     generation inside it), and concurrent calls that do not append and share a
 *     plan are safe. A plan must outlive all work enqueued with it.
 */
#ifndef SEGPAGED_H
#define SEGPAGED_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SEGPAGED_API __attribute__((visibility("default")))

typedef enum {
  SEGPAGED_OK = 0,
  SEGPAGED_EINVAL = -1,        /* invalid argument (null/misaligned pointer, bad spec value) */
  SEGPAGED_EUNSUPPORTED = -2,  /* valid but not supported by the library (head_dim, page size, group) */
  SEGPAGED_ENOSPACE = -3,      /* pool capacity, free list, table or workspace too small */
  SEGPAGED_EHIP = -4,          /* a HIP runtime call or kernel launch failed */
  SEGPAGED_ESTATE = -5         /* call does not fit the plan (e.g. layer out of range) */
} segpaged_status;

/* Head classes, one per (layer, KV head) [RT section 2]. All are causal (key j <= query i).
 *   GLOBAL      every earlier token
 *   LOCAL       the first `sink` tokens and the `window` most recent ones
 *               (j < sink  or  i - window < j), the current token included
 *   RETRIEVAL   only a given sorted set of token positions
 *   DENSE       attends like GLOBAL (its RoPE re-alignment is outside attention) */
typedef enum {
  SEGPAGED_GLOBAL = 0,
  SEGPAGED_LOCAL = 1,
  SEGPAGED_RETRIEVAL = 2,
  SEGPAGED_DENSE = 3
} segpaged_kind;

/* What to plan. All pointers are HOST memory and are read only during
 * segpaged_plan_create. Units are u = (l * num_seqs + b) * num_kv_heads + h. */
typedef struct {
  int32_t num_seqs;             /* B >= 1 */
  int32_t num_layers;           /* >= 1 */
  int32_t num_q_heads;          /* Hq, a multiple of num_kv_heads */
  int32_t num_kv_heads;         /* Hkv >= 1; query head hq reads KV head hq / (Hq/Hkv) [KV 5.3] */
  int32_t head_dim;             /* D in {64, 128} */
  int32_t page_size;            /* P in {16, 32, 64, 128} tokens per page */
  const int32_t* seq_len;       /* [B]  N_b >= 0 tokens in the cache, current token included */
  const int32_t* first_query_pos; /* [B] q0_b in [0, max(N_b-1, 0)]: lowest query position that
                                    will read this table (0 = prefill form, N_b-1 = decode form) */
  const int32_t* kind;          /* [L*Hkv] segpaged_kind, index l * Hkv + h */
  const int32_t* sink;          /* [L*Hkv] sink tokens >= 0 (LOCAL) */
  const int32_t* window;        /* [L*Hkv] window >= 1 (LOCAL) */
  const int64_t* retr_offsets;  /* [U+1] CSR over units into retr_pos; NULL if no RETRIEVAL head */
  const int32_t* retr_pos;      /* sorted unique positions in [0, N_b) per RETRIEVAL unit */
  const int32_t* free_list;     /* page ids in allocation order, NULL = 0, 1, 2, ... */
  int64_t free_list_len;        /* entries in free_list */
  int64_t capacity_pages;       /* pages of the pool the caller provides; 0 = exactly the pages needed.
                                   Every page id must be < capacity. */
  int32_t decode_split_tokens;  /* keys per decode work item, a multiple of 64; 0 = automatic */
  int32_t append_capacity;      /* tokens each sequence may gain after planning; 0 = none */
  int32_t append_chunk;         /* most tokens one append adds to a sequence (with append_capacity;
                                   0 = 1): local heads keep a ring of ceil((W + chunk - 1) / P) + 1
                                   pages, enough for every row of the newest chunk */
  int32_t reserved;             /* 0 */
  /* Document chunks shared by several sequences at the same positions ([SUM]: identical
   * document chunks reuse their KV; [RT section 1]: storage per layer x head x segment):
   * sequences with the same doc_group >= 0 begin with the same doc_len tokens, whose
   * K/V rows are identical in every layer and KV head (the caller's promise; the pool
   * keeps the rows of the group's first sequence). A page whose positions all lie in
   * [0, doc_len) is stored once per (layer, KV head, group) and its id is listed in
   * the page list of every unit that holds the same positions with the same
   * occupancy. Both NULL = no sharing. Not with append_capacity (EUNSUPPORTED). */
  const int32_t* doc_group;     /* [B] group of each sequence, -1 = none */
  const int32_t* doc_len;       /* [B] shared tokens, the same for all members of a group,
                                   <= N_b (0 for sequences without a group) */
} segpaged_spec;

/* Sizes the caller allocates. */
typedef struct {
  int64_t num_pages;        /* distinct pages the table uses (shared document pages once) */
  int64_t pool_pages;       /* pages each pool tensor must hold (= capacity) */
  int64_t pool_bytes;       /* bytes of ONE pool tensor: pool_pages * P * D * 2 */
  int64_t table_int32s;     /* int32 elements of the device table (table + work lists) */
  int64_t table_len;        /* leading int32s that form the SegmentPageTable proper */
  int64_t num_units;        /* L * B * Hkv */
  int64_t q_rows;           /* T_q = sum_b (N_b - q0_b): rows of one layer's Q / O / LSE */
  int64_t kv_rows;          /* T_total = sum_b N_b: rows of one layer's dense K / V */
  int64_t decode_items;     /* decode work items, all layers */
  int64_t prefill_items;    /* prefill work items, all layers */
  int64_t decode_workspace_bytes;  /* workspace for any decode call of the plan, with room
                                      for the extra partials of shared items (see decode) */
  int64_t prefill_workspace_bytes; /* workspace a prefill call needs (0 in this version) */
  int64_t select_workspace_bytes;  /* workspace segpaged_select_topp needs (largest lengths) */
} segpaged_sizes;

/* Algorithmic work of one layer (or all layers when layer = -1), for throughput
 * and roofline accounting. */
typedef struct {
  int64_t units;
  int64_t pages;             /* distinct pages (a page shared by sequences counts once) */
  int64_t retained_tokens;   /* keys stored in the pool, summed over units (padding excluded) */
  int64_t decode_tokens;     /* keys the decode row (position N_b - 1) sees, summed over units */
  int64_t prefill_pairs;     /* visible (query row, key) pairs per KV-head unit over rows q0..N-1;
                                times G gives pairs over Q heads; flops = 4 * D * G * pairs */
  int64_t q_rows;            /* query rows over units (each row serves G query heads) */
  int64_t decode_items;
  int64_t prefill_items;
} segpaged_stats;

typedef struct segpaged_plan segpaged_plan;  /* opaque, host heap */

/* Plan a SegmentPageTable from a spec [RT section 3]: per unit, the retained
 * segments (keys visible to some row >= q0: GLOBAL/DENSE all N; LOCAL the sink
 * and the window reaching back from q0, merged when they touch; RETRIEVAL the
 * given set, gathered), ceil(len / P) pages per segment packed from the segment
 * start, page ids taken in unit/segment/page order from the free list; plus the
 * per-head varlen work lists of the prefill and decode kernels [RT section 4].
 * Host only: makes no HIP call, so it runs without a GPU. The layout is built
 * once here and reused by every call [RT section 5].
 * append_capacity > 0 plans for growth -- a decode loop (chunk 1) or a chunked
 * prefill: each sequence may hold the rows of at most one chunk,
 * N_b - q0_b <= chunk (decode form: q0_b = N_b - 1); global heads reserve the
 * pages of N_b + append_capacity; local heads keep two segments, the sink
 * (ceil(sink/P) pages reserved) and the window [max(sink, q0_b - W + 1), N_b) in
 * a ring of ceil((W + chunk - 1)/P) + 1 pages; the work-list regions and the
 * decode workspace are sized for the largest lengths (see segpaged_plan_append).
 * Returns EINVAL for a bad spec, EUNSUPPORTED for an unsupported D/P/group,
 * ENOSPACE when the free list or capacity is too small. *plan is NULL on error. */
SEGPAGED_API int segpaged_plan_create(const segpaged_spec* spec, segpaged_plan** plan,
                                      segpaged_sizes* sizes);

SEGPAGED_API void segpaged_plan_destroy(segpaged_plan* plan);

SEGPAGED_API int segpaged_plan_sizes(const segpaged_plan* plan, segpaged_sizes* sizes);

/* Host copy of the whole device table image (int32 [table_int32s]). The first
 * table_len ints are the SegmentPageTable, format version 1:
 *   header  16: magic 0x53475054, version 1, B, L, Hq, Hkv, D, P, num_units,
 *               num_pages, num_retr, off_seqs, off_units, off_pages, off_retr, table_len
 *   seqs    4 per sequence: N_b, q0_b, dense K/V row offset, Q row offset
 *   units   16 per unit: class (DENSE stored as GLOBAL), b, l, h, N_b, q0_b, sink,
 *           window, kv_len, nseg, seg0_pos, seg0_len, seg1_pos, seg1_len, page_off,
 *           retr_off (seg0_pos = -1 for a gathered RETRIEVAL segment; retr_off = -1
 *           for other classes; unused segment fields 0)
 *   pages   page id of each table page (a unit's pages start at page_off); an id
 *           repeats where sequences share a document page (doc_group)
 *   retr    positions of the RETRIEVAL segments, units in order
 * The ints after table_len are the build list (num_pages table page slots, in order:
 * the slots that own a distinct page), the kernels' work lists and, last, L + 1
 * lines of 16 zero ints that prefill calls use as work counters (not part of the
 * format; segpaged_build uploads the lines of its layer and of all-layer calls).
 * ENOSPACE if n < table_int32s. */
SEGPAGED_API int segpaged_plan_table_host(const segpaged_plan* plan, int32_t* out, int64_t n);

/* Work counts of one layer (layer = -1: all layers). ESTATE if layer is out of range. */
SEGPAGED_API int segpaged_plan_stats(const segpaged_plan* plan, int32_t layer,
                                     segpaged_stats* stats);

/* build_segpaged_cache [RT section 3]: upload the table slice of `layer` (or the
 * whole table when layer = -1) into d_table, then scatter that layer's retained
 * tokens from dense K/V into their pages:
 *   K page p: bf16 [D/8][P][8], element (slot, d) at ((d/8)*P + slot)*8 + d%8
 *   V page p: bf16 [P/8][D][8], element (slot, d) at ((slot/8)*D + d)*8 + slot%8
 * Unused tail slots are written as zero. Pages of other layers are untouched.
 *   k_dense, v_dense  device bf16 [T_total][Hkv][D] of this layer
 *                     ([L][T_total][Hkv][D] when layer = -1); sequences packed
 *                     in order, sequence b at rows sum_{b'<b} N_b'
 *   d_table           device int32 [table_int32s]
 *   k_pool, v_pool    device bf16, pool_bytes each
 * The upload reads the plan's host memory; keep the plan alive. */
SEGPAGED_API int segpaged_build(const segpaged_plan* plan, int32_t layer,
                                const void* k_dense, const void* v_dense, int32_t* d_table,
                                void* k_pool, void* v_pool, void* stream);

/* Mask-free prefill [RT section 4]: for every query row i in [q0_b, N_b) of every
 * sequence and every Q head hq (KV head h = hq / G):
 *     O = sum_{j in vis(i)} softmax_j(scale * q_i . k_j) v_j,   LSE = log sum exp
 * reading only the pages of (layer, b, h); blocks no row of a tile can see are
 * never read, and no mask tensor exists. Scores and row sums are fp32; the
 * softmax weights enter the P.V products as bf16, except in tiles whose first
 * row sees fewer than 128 keys, where each weight enters as two bf16 terms
 * (hi + lo, ~2^-16 relative): a row with few keys would otherwise carry a
 * weight's bf16 rounding (up to 2^-8 relative) into O almost undiluted.
 *   q     device bf16 [T_q][Hq][D] (rows q0_b..N_b-1 of each sequence, packed in
 *         sequence order); [L][T_q][Hq][D] when layer = -1
 *   o     device bf16, same shape as q (written)
 *   lse   device fp32 [T_q][Hq] natural-log LSE ([L][T_q][Hq] when layer = -1), or NULL
 *   scale softmax scale, typically 1/sqrt(D)
 *   workspace/workspace_bytes: prefill_workspace_bytes (may be NULL when 0)
 * d_table, k_pool, v_pool must hold what segpaged_build wrote for this layer;
 * d_table must be 8-byte aligned here (EINVAL otherwise).
 * Workgroups take the tiles heaviest-first from a 64-bit work counter in d_table's
 * counter line of this layer (layer = -1: the all-layers line), tagged with a
 * generation the plan hands out per call: whatever an earlier launch left there
 * (one that never finished included), the call claims the counter for its own
 * generation and computes every tile; a finished call leaves (generation, 0),
 * so a captured graph of the call also replays. Calls for the same layer on one
 * d_table must not overlap; other calls may.
 * A row whose visible set is empty (RETRIEVAL only) gets O = 0, LSE = -inf. */
SEGPAGED_API int segpaged_prefill(const segpaged_plan* plan, int32_t layer, const void* q,
                                  int32_t* d_table, const void* k_pool,
                                  const void* v_pool, float scale, void* o, float* lse,
                                  void* workspace, int64_t workspace_bytes, void* stream);

/* Growth, host side (the layout is written once, when K/V is written, and then
 * only extended [RT section 5]): every sequence b gains 0 <= n_new[b] <= chunk
 * tokens, N_b += n_new[b]; its rows become the new tokens, q0_b = N_b - n_new[b]
 * (the last row, N_b - 1, when it gains none), so a prefill call computes the
 * newest chunk and a decode call row N_b - 1. Only for plans made with
 * append_capacity > 0 (ESTATE otherwise); ENOSPACE if a sequence would pass its
 * planned length plus append_capacity, EINVAL for a count < 0 or > chunk. Updates
 * the plan's image: sequence rows; unit records (a global head's segment grows
 * into its reserved pages; a local head keeps its sink and the window positions
 * [p0, N) in a ring of ceil((W + chunk - 1)/P) + 1 pages: when it outgrows the ring,
 * p0 moves on by P and the id of the page that held the oldest positions moves
 * to the end of the ring); the work lists; and the append list the next
 * segpaged_append reads. Sizes (table_int32s, pools, workspace) do not change.
 * No HIP call. */
SEGPAGED_API int segpaged_plan_append(segpaged_plan* plan, const int32_t* n_new);

/* Decode-loop growth, device side: write the K/V of the tokens the last
 * segpaged_plan_append added into their pages; the first call after it also
 * uploads the changed parts of the image (all layers) into d_table.
 *   k_new, v_new  device bf16 [T_new][Hkv][D] of this layer, T_new = sum of
 *                 n_new, rows packed in sequence order ([L][T_new][Hkv][D] when
 *                 layer = -1); may be NULL when T_new = 0
 *   d_table, k_pool, v_pool  as built by segpaged_build for this plan
 * Retrieval heads store nothing (their index set is given). Call it for a layer
 * before that layer's decode, on the stream the decode uses. ESTATE for a plan
 * without append capacity or a layer out of range. */
SEGPAGED_API int segpaged_append(segpaged_plan* plan, int32_t layer, const void* k_new,
                                 const void* v_new, int32_t* d_table, void* k_pool,
                                 void* v_pool, void* stream);

/* Retrieval-set selection, top-p by attention mass ([RT] section 2: retrieval
 * heads keep the top-p important tokens, looked up on demand): for every
 * RETRIEVAL KV head h of `layer` and every sequence b, the decode row's (position
 * N_b - 1) attention over all N_b keys of the dense history, averaged over the G
 * query heads of the group, is the mass of each key; the selected set is the
 * shortest prefix of the keys ordered by mass (larger first, equal masses by
 * position) whose mass reaches p of the total, as sorted positions. It is the
 * retrieval set a new plan (segpaged_spec.retr_pos) then keeps.
 *   q        device bf16 [B][Hq][D]: the decode row of each sequence
 *   k_dense  device bf16 [T_total][Hkv][D] of this layer (sequences packed in order)
 *   d_table  as built for this plan (sequence lengths and head classes)
 *   scale    softmax scale; p in (0, 1]
 *   out_pos  device int32 [Hkv][T_total]: the set of (b, h) at h * T_total +
 *            (first dense row of b), out_cnt[b * Hkv + h] entries
 *   out_cnt  device int32 [B * Hkv] (0 for other classes and empty sequences)
 *   workspace/workspace_bytes: select_workspace_bytes
 * Sums run in a fixed order, so repeated calls return the same set; where fp32
 * rounding of the masses decides between keys of nearly equal mass the set may
 * differ from an exact computation in those keys only. EINVAL / ENOSPACE / ESTATE
 * (layer = -1 is not accepted) as above. */
SEGPAGED_API int segpaged_select_topp(const segpaged_plan* plan, int32_t layer, const void* q,
                                      const void* k_dense, const int32_t* d_table, float scale,
                                      float p, int32_t* out_pos, int32_t* out_cnt, void* workspace,
                                      int64_t workspace_bytes, void* stream);

/* The pages of `layer` (every layer when -1) as one contiguous stream per tensor,
 * for moving a cache to another device or process: prefill and decode on separate
 * machines move KV between them, and a SegPaged cache moves only what each head
 * keeps [SUM: KV transfer bytes in the disaggregated setting]. The stream holds the
 * distinct pages of that range in table order of first use (a shared document page
 * once), each in the pool page layout of segpaged_build: stats(layer).pages * P * D
 * bf16 per tensor (tail slots included).
 *   d_table  device table image uploaded by segpaged_build or segpaged_import_pages
 *   k_out, v_out  device bf16 streams (written); pools are only read
 * The stream depends on the plan's units and segments, not on its page ids. */
SEGPAGED_API int segpaged_export_pages(const segpaged_plan* plan, int32_t layer,
                                       const int32_t* d_table, const void* k_pool,
                                       const void* v_pool, void* k_out, void* v_out,
                                       void* stream);

/* The inverse: upload the table slice of `layer` (as segpaged_build does), then write
 * the streamed pages into this plan's pages. The plan must come from the same spec as
 * the exporting plan up to free list and pool capacity, so its units, segments and
 * page counts match; its page ids may differ. Pages of other layers are untouched.
 *   k_in, v_in  device bf16 streams of stats(layer).pages * P * D elements each */
SEGPAGED_API int segpaged_import_pages(const segpaged_plan* plan, int32_t layer,
                                       const void* k_in, const void* v_in, int32_t* d_table,
                                       void* k_pool, void* v_pool, void* stream);

/* Split-K decode [RT section 4; KV section 10.2]: the query at position N_b - 1 of
 * each sequence attends to every key it can see. Work items are (unit, key
 * range) slices; each writes fp32 partials (running max, normaliser, unnormalised
 * output) for the G query heads of its unit into `workspace`, and a combine pass
 * merges them with the log-sum-exp rule into O and LSE. The softmax weights enter
 * the P.V products as two bf16 terms each (hi + lo, ~2^-16 relative).
 *   q     device bf16 [B][Hq][D] ([L][B][Hq][D] when layer = -1)
 *   o     device bf16, same shape (written)
 *   lse   device fp32 [B][Hq] ([L][B][Hq]), or NULL
 *   workspace  device memory for the call's partials: one record of G * (D + 4) floats
 *              per item of the call at least (ENOSPACE otherwise); decode_workspace_bytes
 *              is enough for any call of the plan
 * Works on any plan form; a decode-form plan (q0 = N-1) stores only what the row sees.
 * Items may be shared by several waves, each writing its own partial, as long as a
 * wave keeps >= 256 keys and workspace_bytes holds the extra partials. A launch with
 * fewer items than the device holds decode waves at once (2048 on an MI355X; one
 * layer of a plan whose split was sized for all its layers) deals each item's keys
 * to up to 16 waves, as many as fit in that one round: the all-layer workspace of a
 * plan of >= 16 layers holds them for any of its layers. A launch of several rounds
 * deals its last items, one round of waves' worth (up to 512), to 4 waves each, so
 * that it ends on short waves; decode_workspace_bytes includes those 1536 partials. */
SEGPAGED_API int segpaged_decode(const segpaged_plan* plan, int32_t layer, const void* q,
                                 const int32_t* d_table, const void* k_pool, const void* v_pool,
                                 float scale, void* o, float* lse, void* workspace,
                                 int64_t workspace_bytes, void* stream);

/* segpaged_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, serving loops and harnesses that forbid hipMalloc): the same
 * computation, with the decode workspace taken from a library-owned device array
 * of SEGPAGED_NOALLOC_SCRATCH_BYTES, one per GPU, held until the process ends
 * (looked up on a device at its first call there). Makes no allocation of any kind.
 * A call whose partials need more than that array returns ENOSPACE before any work
 * is enqueued (a call over one layer of the Llama-3.3-70B-shaped 8 x 32K decode
 * needs ~15 MB; the array also decides how many waves share an item, exactly as a
 * workspace_bytes of that size does). Calls that overlap on one GPU share the array
 * and race: serialise them (one stream, or events). The array needs no clearing:
 * every partial a call reads was written by that call. */
#define SEGPAGED_NOALLOC_SCRATCH_BYTES (32LL << 20)
SEGPAGED_API int segpaged_decode_noalloc(const segpaged_plan* plan, int32_t layer, const void* q,
                                         const int32_t* d_table, const void* k_pool,
                                         const void* v_pool, float scale, void* o, float* lse,
                                         void* stream);

SEGPAGED_API const char* segpaged_status_str(int status);

/* Library version: major * 10000 + minor * 100 + patch. */
SEGPAGED_API int segpaged_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SEGPAGED_H */
