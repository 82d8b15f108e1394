/*
 * pkvt.h -- C ABI of libpkvt: decode-time self-attention over a prefix-tree
 * KV cache, computed as a two-phase partition, for AMD Instinct MI355X
 * (gfx950).
 *
 * Source of the method: "ChunkAttention: Efficient Self-Attention with
 * Prefix-Aware KV Cache and Two-Phase Partition" (Ye, Tao, Huang, Li; ACL
 * 2024), as digested on its chapterpal page:
 *   Knowl 1 -- prefix-aware KV cache: KV sliced into chunks of c tokens that
 *              are nodes of a prefix tree; arrival / decode / departure; pool
 *              allocator with a free list.
 *   Knowl 2 -- the two-phase partition (TPP) decode algorithm.
 *   Knowl 3 -- partial_attn and attn_reduce (online softmax) equations.
 *   Knowl 5 -- context tuples (C, i, j) sent to the GPU, lazy context copy.
 * The 1/sqrt(d) score scale is the attention definition's (CachedAttention
 * digest, "Load-bearing equations"); callers pass it explicitly.
 *
 * Conventions
 *   - Every function returns pkvt_status: 0 on success, a negative code on
 *     failure.  Nothing throws across the ABI.  pkvt_last_error() returns a
 *     thread-local message describing the last failure on the calling thread.
 *   - A pkvt_tree is host state owned by the library (create/destroy).  It is
 *     not thread-safe: use one host thread per tree at a time.
 *   - All DEVICE memory (K/V pools, Q, O, metadata, workspace, slot arrays
 *     for the scatter) is allocated and owned by the caller and passed as
 *     raw device pointers.  The library never allocates device memory; its
 *     only device storage is the fixed scratch array of
 *     pkvt_attn_decode_noalloc, part of the loaded code object.
 *   - "stream" arguments are hipStream_t values passed as void*; NULL is the
 *     default stream.  Device work is asynchronous on that stream.
 *   - Host pointer arguments are only read/written during the call.
 *   - Mutating calls that fail leave the tree exactly as it was.
 *
 * Shapes: n_heads h (query heads == KV heads), all tensors fp16 (IEEE
 * binary16).  The kernels support head_dim d in {64, 128, 256} and chunk_size c
 * in {16, 32, 64, 128}; the host tree and planner accept any c in [1, 4096]
 * and d >= 1, and the device entry points (pkvt_pool_bytes, pkvt_kv_scatter,
 * pkvt_plan_upload, pkvt_attn_decode) return UNSUPPORTED_SHAPE otherwise.
 */
#ifndef PKVT_H
#define PKVT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t pkvt_status;

#define PKVT_OK                     0
#define PKVT_ERR_INVALID_ARG       -1  /* bad pointer, size, id list, or option            */
#define PKVT_ERR_NO_CHUNKS         -2  /* chunk pool exhausted (nothing was changed)        */
#define PKVT_ERR_UNKNOWN_SEQ       -3  /* sequence id is not live                           */
#define PKVT_ERR_EMPTY_SEQ         -4  /* a sequence with zero tokens                       */
#define PKVT_ERR_UNSUPPORTED_SHAPE -5  /* head_dim / chunk_size outside the supported set   */
#define PKVT_ERR_BUFFER_TOO_SMALL  -6  /* caller buffer smaller than required               */
#define PKVT_ERR_STALE_PLAN        -7  /* no plan, plan older than the tree, or not uploaded */
#define PKVT_ERR_HIP               -8  /* a HIP runtime call or kernel launch failed        */
#define PKVT_ERR_HOST_MEMORY       -9  /* host allocation failed                            */

typedef struct pkvt_tree pkvt_tree;

/* ------------------------------------------------------------------------
 * Device chunk pool (Knowl 1: each tree node owns one chunk holding the K
 * and V slices, h x c x d each, of its c tokens).
 *
 * A chunk id n in [0, pool_chunks) addresses one slice of h*c*d halves in
 * the K pool and one in the V pool, at element offset n*h*c*d.  Within a
 * chunk, head j's slice starts at j*c*d and is laid out for the gfx950
 * matrix cores, not as a plain [c][d] matrix:
 *   K slice: [d/8][c][8]  -- element (token t, dim x) at ((x/8)*c + t)*8 + x%8
 *   V slice: blocks of F tokens one after the other, F = 32 (16 when
 *            head_dim is 256 or c is 16); a block is [d/16][F/8][16][8]:
 *            element (token t, dim x), with w = t%F, at
 *              (t-w)*d + (((x/16)*(F/8) + g)*16 + x%16)*8 + e
 *            where for F = 32: g = (w%16)/4, e = (w/16)*4 + w%4 (tokens
 *            4g..4g+3 and 16+4g..16+4g+3 share one 8-element run, the
 *            operand order of the matrix cores), and for F = 16: g = w/8,
 *            e = w%8
 * Callers never compute these offsets: pkvt_kv_scatter writes tokens given
 * in natural [token][head][dim] order.  pkvt_pool_bytes gives the size of
 * ONE pool (K or V) for one layer.
 * ---------------------------------------------------------------------- */
pkvt_status pkvt_pool_bytes(int32_t n_heads, int32_t head_dim, int32_t chunk_size,
                            int32_t pool_chunks, size_t* bytes);

/* ------------------------------------------------------------------------
 * Host prefix tree (Knowl 1).
 * ---------------------------------------------------------------------- */

/* Create an empty tree over a pool of pool_chunks chunks (all free).
 * INVALID_ARG if n_heads < 1, head_dim < 1, chunk_size outside [1, 4096],
 * pool_chunks < 1 or out is NULL. */
pkvt_status pkvt_tree_create(int32_t n_heads, int32_t head_dim, int32_t chunk_size,
                             int32_t pool_chunks, pkvt_tree** out);
void        pkvt_tree_destroy(pkvt_tree* tree);

/* pkvt_tree_create with a choice of prefix matching:
 *   PKVT_MATCH_CHUNKS -- whole-chunk matching (Knowl 1's nodes are whole
 *                        chunks); what pkvt_tree_create gives.
 *   PKVT_MATCH_TOKENS -- token-granular matching, a variant the page does not
 *                        describe: an arrival shares its longest common token
 *                        prefix with the tree even when that prefix ends
 *                        inside a chunk.  A node then holds 1..c tokens at the
 *                        start of its chunk.  The arrival descends into the
 *                        child whose tokens share the longest prefix with the
 *                        rest of its prompt (ties: the earliest created) and
 *                        SPLITS a child it matches only in part: the child
 *                        keeps the matched tokens, a new node (a new chunk)
 *                        below it takes the rest and the old children.  The
 *                        K/V of those tokens must then move: see
 *                        pkvt_tree_moves / pkvt_kv_move.  A decode append
 *                        writes into the leaf only while that leaf is partial,
 *                        private and childless, else it opens a new leaf.
 *                        Nodes are never merged.  The planners and kernels
 *                        (decode and prefill) accept such trees: a work item
 *                        ends at every partial chunk.
 * INVALID_ARG also for any other match value. */
#define PKVT_MATCH_CHUNKS 0
#define PKVT_MATCH_TOKENS 1
pkvt_status pkvt_tree_create_ex(int32_t n_heads, int32_t head_dim, int32_t chunk_size,
                                int32_t pool_chunks, int32_t match, pkvt_tree** out);

/* Sequence arrival (Knowl 1): insert n_seqs prompts.
 *   tokens  : int32 token ids of all prompts, concatenated.
 *   offsets : int64 [n_seqs+1]; prompt s is tokens[offsets[s] .. offsets[s+1]).
 * Matching is whole-chunk from token 0: the longest run of FULL chunks whose
 * c tokens (and therefore whole prefix) equal an existing full chunk on the
 * path is shared (refcount + 1); the remaining tokens are stored in newly
 * allocated chunks, inserted as a branch; a partial last chunk is private.
 * (Token matching, pkvt_tree_create_ex: the longest common token prefix is
 * shared, splitting a node where it ends inside one; slots are then final
 * positions after every split of the call, and the K/V of tokens stored
 * before the call that a split relocated are listed by pkvt_tree_moves.)
 * Prompts inserted earlier in the same call can be matched by later ones.
 * Outputs:
 *   seq_ids : int32 [n_seqs], the new sequences' ids (never reused).
 *   slots   : int64 [offsets[n_seqs]]; for each token, chunk_id*c + position
 *             in the chunk where the caller must store that token's K/V, or
 *             -1 when the token lives in a chunk that already existed.
 * Errors: EMPTY_SEQ (a prompt of length 0), NO_CHUNKS (pool exhausted),
 * INVALID_ARG.  All-or-nothing: on error no sequence is inserted. */
pkvt_status pkvt_tree_build(pkvt_tree* tree, int32_t n_seqs, const int32_t* tokens,
                            const int64_t* offsets, int32_t* seq_ids, int64_t* slots);

/* Decode append (Knowl 1): token i goes to sequence seq_ids[i]'s leaf chunk
 * until that chunk is full, then to a new private leaf chunk (under token
 * matching also when the leaf is shared or has children).  Several
 * entries may name the same sequence; they are applied in order.
 * slots[i] receives chunk_id*c + position for token i (never -1).
 * Errors: UNKNOWN_SEQ, NO_CHUNKS, INVALID_ARG.  All-or-nothing. */
pkvt_status pkvt_tree_append(pkvt_tree* tree, int32_t n, const int32_t* seq_ids,
                             const int32_t* tokens, int64_t* slots);

/* Sequence departure (Knowl 1): drop the sequence from its path; chunks no
 * live sequence uses any more return to the free list (pool memory is kept)
 * and their nodes are pruned.  Errors: UNKNOWN_SEQ. */
pkvt_status pkvt_tree_remove(pkvt_tree* tree, int32_t seq_id);

/* Introspection (tests, accounting). */
typedef struct {
    int32_t capacity;       /* pool_chunks                                    */
    int32_t used_chunks;    /* chunks owned by live nodes                     */
    int32_t free_chunks;    /* capacity - used_chunks                         */
    int32_t shared_chunks;  /* live chunks with refcount >= 2                 */
    int32_t live_seqs;
    int32_t reserved[3];
} pkvt_stats;
pkvt_status pkvt_tree_stats(const pkvt_tree* tree, pkvt_stats* out);
/* Chunk ids of the sequence's root-to-leaf path.  *n receives the path
 * length; at most cap ids are written (BUFFER_TOO_SMALL if cap < *n). */
pkvt_status pkvt_tree_chunk_path(const pkvt_tree* tree, int32_t seq_id, int32_t* ids,
                                 int32_t cap, int32_t* n);
/* Number of tokens currently stored for the sequence. */
pkvt_status pkvt_tree_seq_len(const pkvt_tree* tree, int32_t seq_id, int64_t* len);
/* Live sequences through the chunk (0 for a free chunk). */
pkvt_status pkvt_tree_chunk_refcount(const pkvt_tree* tree, int32_t chunk_id, int32_t* refs);
/* Tokens stored in the chunk (0 for a free chunk; below c only for a leaf
 * under whole-chunk matching, anywhere under token matching). */
pkvt_status pkvt_tree_chunk_fill(const pkvt_tree* tree, int32_t chunk_id, int32_t* fill);

/* K/V moves made necessary by the most recent pkvt_tree_build (token
 * matching; always none under whole-chunk matching): the token whose K/V is
 * at slot src[i] now belongs at slot dst[i] (slot = chunk_id*c + position).
 * Sources lie in chunks that existed before that build, destinations in
 * chunks it allocated, so the two sets are disjoint, and none of them is a
 * slot the build returned for a new token: apply the moves (pkvt_kv_move,
 * once per layer's pools) and write the new tokens in either order, both
 * before the next attention call.  *n receives the number of moves; at most
 * cap are written (BUFFER_TOO_SMALL if cap < *n, so cap 0 with NULL src/dst
 * asks for the count).  The list is replaced by every pkvt_tree_build call. */
pkvt_status pkvt_tree_moves(const pkvt_tree* tree, int64_t* src, int64_t* dst, int64_t cap,
                            int64_t* n);

/* ------------------------------------------------------------------------
 * Plan = context generation (Knowl 5): the host walks the tree and emits the
 * work of both phases for one decode batch.
 *
 * The batch's query rows are q_order[0..b): row r of Q and O belongs to
 * sequence q_order[r] (distinct live ids, each with >= 1 token).
 * Sequences are renumbered in depth-first leaf order so that the batch
 * sequences covered by any node form one contiguous range [i, j) (Knowl 1's
 * contiguity invariant); a node with j - i >= min_share is "shared" and goes
 * to phase 1 (Knowl 2: chunks covered by multiple sequences), where chains
 * of consecutive shared nodes with the same [i, j) are cut into work items of
 * at most phase1_chunks chunks -- each item is one context tuple (chunk list,
 * i, j).  Every other chunk is processed per sequence in phase 2, cut into
 * items of at most phase2_chunks chunks.  Each (item, group of 16 query
 * rows, head) is one task of a 64-lane wave; the attention kernel runs a
 * fixed grid of persistent workgroups of 4 waves and every wave walks a task
 * list filled longest-first by the planner (the row groups of one phase-1
 * item share a workgroup, so its chunks are fetched once per CU).  By
 * default items are cut at the mean per-wave load, so no task is longer
 * than what a perfectly balanced wave would do.
 *
 * Re-planning the same batch (same q_order and options) is lazy (Knowl 5):
 * when only sequence lengths changed, only the length table is rewritten;
 * when the only structural changes since the last plan are decode appends
 * that opened new leaf chunks, each such chunk is added to the end of its
 * row's last (sequence-first) work item, in room the plan keeps there, and
 * nothing else is re-planned; any other change (an arrival, a departure, a
 * row whose room is used up or whose path ends in shared chunks, or 256
 * patches in a row) builds the plan afresh.
 * ---------------------------------------------------------------------- */
typedef struct {
    int32_t phase1_chunks;  /* max chunks per phase-1 item; 0 = derived from
                               the mean per-wave load (see below)             */
    int32_t phase2_chunks;  /* max chunks per phase-2 item; 0 = derived       */
    int32_t min_share;      /* 0 = default 2.  A value above b disables phase 1:
                               every chunk is read per sequence (plain paged
                               decode over shared physical chunks).           */
    int32_t workgroups;     /* persistent workgroups of the attention kernel;
                               0 = 2 per compute unit of the current device
                               (512 when no device is visible)                */
    int32_t unit_rows;      /* smallest phase-1 row block run as a workgroup
                               unit (LDS-shared loads); 0 = default 17.  A
                               value above 64 runs every phase-1 row group
                               as a single-wave task.                         */
} pkvt_plan_opts;

typedef struct {
    int32_t b;
    int32_t phase1_items;   /* context tuples (chunk segment, i, j)            */
    int32_t phase2_items;
    int32_t waves;          /* wave descriptors (item x row group)             */
    int32_t workgroups;     /* persistent workgroups of the attention kernel   */
    int32_t slots;          /* partial results per head in the workspace       */
    int32_t merge_rows;     /* sequences whose partials are merged             */
    int32_t shared_chunks;  /* distinct chunks read in phase 1                 */
    int64_t unique_tokens;  /* valid tokens in distinct chunks of the batch    */
    int64_t logical_tokens; /* sum of the batch's sequence lengths             */
    int32_t structure_version;
    int32_t tasks;          /* wave tasks (waves x heads)                      */
    int32_t phase1_split;   /* chunks per phase-1 item actually used           */
    int32_t phase2_split;   /* chunks per phase-2 item actually used           */
    int32_t wg_units;       /* workgroup units: phase-1 row blocks of 17..64
                               rows whose 4 waves share every K/V load through
                               LDS                                             */
    int32_t last_update;    /* what the last pkvt_plan call did: 0 refreshed
                               the sequence lengths only, 1 patched the plan
                               for decode appends that opened new leaf chunks,
                               2 built it afresh                               */
    int32_t patches;        /* patches since the plan was last built           */
    int32_t kernel;         /* 0: the two-phase kernel (workgroup units and
                               single-wave tasks, 2 workgroups of 4 waves per
                               compute unit); 1: the units-only kernel, chosen
                               when every row's context lies in chunks shared
                               by at least unit_rows rows and head_dim >= 128
                               (one workgroup of 8 waves per compute unit:
                               two groups of 4 waves take alternate steps of
                               each unit, so two steps are in flight)          */
} pkvt_plan_info;

/* Build the plan for a batch.  opts may be NULL (defaults).  Reports the
 * device byte sizes the caller must provide: meta_bytes for the metadata
 * buffer (pkvt_plan_upload) and workspace_bytes for pkvt_attn_decode (fp32
 * partial results; 0 when nothing needs merging).  Errors: UNKNOWN_SEQ,
 * EMPTY_SEQ, INVALID_ARG (b < 1, duplicate ids, bad options). */
pkvt_status pkvt_plan(pkvt_tree* tree, int32_t b, const int32_t* q_order,
                      const pkvt_plan_opts* opts, size_t* meta_bytes,
                      size_t* workspace_bytes);
pkvt_status pkvt_plan_info_get(const pkvt_tree* tree, pkvt_plan_info* out);
/* Introspection for tests: copy the current plan's int32 metadata blob (the
 * exact words pkvt_plan_upload sends) to out.  *n receives its length in
 * words; BUFFER_TOO_SMALL if cap < *n (nothing copied).  The layout is
 * internal to the library and versioned by its first word. */
pkvt_status pkvt_plan_blob(const pkvt_tree* tree, int32_t* out, int32_t cap, int32_t* n);

/* Copy the current plan to the caller's device buffer d_meta (>= meta_bytes)
 * asynchronously on stream: the words go to a pinned, device-mapped host
 * staging buffer and a small kernel on stream copies them into d_meta (no
 * copy engine is involved).  Lazy (Knowl 5): when d_meta already holds this
 * plan nothing is copied, and when only sequence lengths changed (decode
 * appends that did not open a new chunk) only the length table is copied.
 * The library keeps a ring of 4 staging buffers and reuses one only after
 * the copy from it has run, so the host may run up to 4 uploads ahead.
 * Errors: STALE_PLAN (no plan / tree changed since pkvt_plan),
 * BUFFER_TOO_SMALL, HIP. */
pkvt_status pkvt_plan_upload(pkvt_tree* tree, void* d_meta, size_t meta_bytes, void* stream);

/* Decode attention for the planned batch (Knowl 2), on stream:
 *   q        : device fp16 [b][h][d], row r = sequence q_order[r]
 *   k_pool,
 *   v_pool   : device fp16 pools (layout above); the caller may pass the pools
 *              of any layer that shares this tree
 *   out      : device fp16 [b][h][d]; O[r] = softmax(scale * q_r K^T) V over
 *              every token stored for sequence q_order[r]
 *   d_meta   : the buffer given to pkvt_plan_upload for the current plan
 *   workspace: device buffer of >= workspace_bytes (contents need not be
 *              initialised; it is scratch for this call only)
 *   scale    : score scale, normally 1/sqrt(d)
 * Phase 1 (chunk-first, matrix cores) and phase 2 (sequence-first) run in one
 * launch and leave unnormalised partials (o, m, n) in the workspace; a merge
 * launch folds them with attn_reduce (Knowl 3) and divides.  Sequences with
 * a single partial are finalised in place and skip the merge.
 * Errors: STALE_PLAN (plan not current or not uploaded to d_meta),
 * BUFFER_TOO_SMALL, INVALID_ARG, HIP. */
pkvt_status pkvt_attn_decode(const pkvt_tree* tree, const void* d_meta, const void* q,
                             const void* k_pool, const void* v_pool, void* out,
                             void* workspace, size_t workspace_bytes, float scale,
                             void* stream);

/* pkvt_attn_decode with profiling hooks: attn_start_event and
 * attn_end_event, when not NULL, must be hipEvent_t values (passed as void*)
 * created on the current device; they are recorded on stream right before
 * the attention kernel is queued and right after it (before the merge
 * kernel), so that the caller can time the attention kernel alone with
 * events on the same stream.  Same arguments and errors as pkvt_attn_decode
 * otherwise. */
pkvt_status pkvt_attn_decode_ex(const pkvt_tree* tree, const void* d_meta, const void* q,
                                const void* k_pool, const void* v_pool, void* out,
                                void* workspace, size_t workspace_bytes, float scale,
                                void* stream, void* attn_start_event, void* attn_end_event);

/* pkvt_attn_decode for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels, with the partial results in a fixed device
 * scratch array of PKVT_NOALLOC_SCRATCH_BYTES (64 MiB) that the library
 * holds on every device it runs on until the process ends, instead of a
 * caller workspace.  The call allocates nothing.  Arguments as
 * pkvt_attn_decode, less the workspace; the current device must be the one
 * that q, the pools and out live on.  The scratch is shared by every call
 * on a device and keeps the last call's contents (nothing in it needs to
 * start at zero): calls that overlap on one device -- on different
 * streams, or from several host threads -- race on it and must not be
 * issued.  Errors: BUFFER_TOO_SMALL when the plan's partials
 * (workspace_bytes of pkvt_plan) exceed the scratch, otherwise as
 * pkvt_attn_decode. */
#define PKVT_NOALLOC_SCRATCH_BYTES (64u << 20)
pkvt_status pkvt_attn_decode_noalloc(const pkvt_tree* tree, const void* d_meta, const void* q,
                                     const void* k_pool, const void* v_pool, void* out,
                                     float scale, void* stream);

/* ------------------------------------------------------------------------
 * Prefix-aware prefill (Knowl 1 arrival: matched prefix chunks are shared,
 * the newly computed suffix tokens are stored in new chunks).  After a
 * pkvt_tree_build (or appends, for a prompt fed in pieces) and
 * pkvt_kv_scatter of the new tokens' K/V, the new tokens' queries attend
 * causally: the row at position p of sequence s sees s's tokens 0 .. p, the
 * stored prefix included.  Chunks that several batch sequences read are
 * read once per block of up to 256 rows (128 at head_dim 256) for all of
 * them together (the chunk-first phase of Knowl 2 applied to many query
 * rows).
 * ---------------------------------------------------------------------- */

/* Plan the prefill of n sequences: query rows are positions q_from[i] ..
 * len_i - 1 of sequence seq_ids[i], sequences in the given order, positions
 * ascending (R rows in all).  opts may be NULL; phase1_chunks caps the
 * chunks per work item (0 = 128, also the maximum), workgroups sets the
 * grid (0 = as for pkvt_plan, two per compute unit: a prefill workgroup has
 * 8 waves and one is resident per compute unit, so the second half starts
 * as the first finishes), the other fields are ignored.  Reports the metadata bytes (pkvt_prefill_upload) and
 * the workspace bytes (fp32 partials) pkvt_prefill_attn needs.
 * Errors: UNKNOWN_SEQ, INVALID_ARG (n < 1, a duplicate id, q_from outside
 * [0, len)), HOST_MEMORY. */
pkvt_status pkvt_prefill_plan(pkvt_tree* tree, int32_t n, const int32_t* seq_ids,
                              const int64_t* q_from, const pkvt_plan_opts* opts,
                              size_t* meta_bytes, size_t* workspace_bytes);
/* Summary of the prefill plan (b = R rows, slots = partials, wg_units =
 * work units; the decode-only fields are 0). */
pkvt_status pkvt_prefill_info_get(const pkvt_tree* tree, pkvt_plan_info* out);
/* Introspection for tests: the prefill plan's metadata words, as
 * pkvt_plan_blob. */
pkvt_status pkvt_prefill_blob(const pkvt_tree* tree, int32_t* out, int32_t cap, int32_t* n);
/* Copy the prefill plan to d_meta, as pkvt_plan_upload does for the decode
 * plan (skipped when d_meta already holds it).  A d_meta buffer holds one
 * plan at a time: uploading either plan into it makes the other stale.
 * Errors: STALE_PLAN, BUFFER_TOO_SMALL, UNSUPPORTED_SHAPE, HIP. */
pkvt_status pkvt_prefill_upload(pkvt_tree* tree, void* d_meta, size_t meta_bytes, void* stream);
/* Prefill attention on stream:
 *   q   : device fp16 [R][h][d], rows as pkvt_prefill_plan numbers them
 *   out : device fp16 [R][h][d]
 *   k_pool, v_pool : the layer's pools, holding every token of the batch
 *         sequences (the new ones written by pkvt_kv_scatter beforehand)
 *   workspace : device, >= workspace_bytes of pkvt_prefill_plan (may be NULL
 *         when that is 0: every row is then written by a single work unit)
 * One attention launch (work units only) and, when some row has several
 * partials, one merge launch.
 * Errors: INVALID_ARG, STALE_PLAN (no prefill plan for the current tree, or
 * not uploaded to d_meta), BUFFER_TOO_SMALL, UNSUPPORTED_SHAPE, HIP. */
pkvt_status pkvt_prefill_attn(const pkvt_tree* tree, const void* d_meta, const void* q,
                              const void* k_pool, const void* v_pool, void* out,
                              void* workspace, size_t workspace_bytes, float scale, void* stream);

/* Write n_tokens tokens' K/V into the pools (the caller's side of arrival
 * and decode append):
 *   slots : device int64 [n_tokens] from pkvt_tree_build / pkvt_tree_append;
 *           entries outside [0, pool_chunks*c) (such as the -1 of tokens
 *           already stored) are skipped.
 *   k_new, v_new : device fp16 [n_tokens][h][d], natural order.
 * Errors: INVALID_ARG, HIP. */
pkvt_status pkvt_kv_scatter(const pkvt_tree* tree, void* k_pool, void* v_pool,
                            const int64_t* slots, const void* k_new, const void* v_new,
                            int64_t n_tokens, void* stream);

/* pkvt_kv_scatter for one decode step's new tokens with the slots still in
 * HOST memory (as pkvt_tree_append returned them): the n_tokens <=
 * PKVT_INLINE_SLOTS slots are copied into the kernel's launch arguments
 * during the call, so the caller needs no device slot buffer and the stream
 * no host-to-device copy.  slots may be reused as soon as the call returns.
 * Errors: INVALID_ARG (also n_tokens > PKVT_INLINE_SLOTS), HIP. */
#define PKVT_INLINE_SLOTS 256
pkvt_status pkvt_kv_scatter_host_slots(const pkvt_tree* tree, void* k_pool, void* v_pool,
                                       const int64_t* slots, const void* k_new,
                                       const void* v_new, int64_t n_tokens, void* stream);

/* Move n tokens' K/V inside one layer's pools: slot src[i] -> slot dst[i],
 * all heads (the moves of pkvt_tree_moves).
 *   src, dst : device int64 [n]; pairs with an entry outside
 *              [0, pool_chunks*c) are skipped.  The source and destination
 *              slot sets must be disjoint (pkvt_tree_moves' are).
 * Errors: INVALID_ARG, UNSUPPORTED_SHAPE, HIP. */
pkvt_status pkvt_kv_move(const pkvt_tree* tree, void* k_pool, void* v_pool, const int64_t* src,
                         const int64_t* dst, int64_t n, void* stream);

const char* pkvt_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* PKVT_H */
