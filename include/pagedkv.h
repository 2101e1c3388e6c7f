/*
 * pagedkv.h -- C ABI of libpagedkv.so: K/V append and varlen decode attention
 * over a paged KV cache or a column-packed ring store, and the prefix copies
 * between a dense prefill cache and the paged one, for AMD gfx950.
 *
 * Sources of the operations (pages, by title and section):
 *  - vLLM-Omni "paged_decode" (SenseNova-U1), PagedDecodeCache class docstring
 *    and PagedDecodeCache.attend: per-layer K/V laid out
 *    (num_blocks, BLOCK_SIZE = 16, kv_heads, head_dim), read through a block
 *    table; the live length (seqused_k) and the write slot live in device
 *    tensors so one captured graph serves every length in a bucket; append this
 *    step's K/V, then attend over the whole valid prefix with
 *    flash_attn_varlen_func(max_seqlen_q, cu_seqlens_q, max_seqlen_k,
 *    seqused_k, block_table, softmax_scale, causal).
 *  - ExecuTorch PR #24073 "Add a batched-sequence CUDA KV cache" (the
 *    sdpa_varlen and lowering parts): a [rows, cols, H, D] column store, a device
 *    segment table seq_info Int32[S, 4] = (q_start, q_len, col, kv_end), causal
 *    and non-causal, sliding window over ring storage, GQA, rows no segment
 *    covers zeroed, split-K for short steps; in-graph writes to slot
 *    (position % rows) * columns + column.
 *  - tiny-llm kv_cache.py, causal_kwargs: with T new queries over start + T
 *    keys, query i sees keys 0 .. start + i; padded_causal_mask: keys before a
 *    row's first valid position are hidden, the diagonal always kept.
 *
 * Conventions for every call:
 *  - All pointers are DEVICE pointers unless stated.  The caller owns every
 *    buffer; the library never allocates, frees, synchronises or reads device
 *    memory from the host, and keeps no pointer after a call returns.  Work is
 *    enqueued on `stream` (a hipStream_t; NULL is the default stream), so every
 *    call may be captured into a hipGraph.  The launch geometry depends only on
 *    host arguments: lengths, tables and slots are read on the device.
 *  - Tensors are dense and row-major.  q, K, V, k_new, v_new and out share one
 *    element type (`dtype`); accumulation is fp32; out is rounded to nearest-even.
 *  - Host-checkable argument errors return before anything is enqueued:
 *    PKV_EINVAL (null pointer, non-positive size, q_heads % kv_heads != 0,
 *    head_dim % 8 != 0 or head_dim > 256, block_size != 16, both or neither
 *    addressing mode, num_segments > 2 * cols, a window with ring storage that
 *    cannot hold window + max_seqlen_q - 1 rows), PKV_EUNSUPPORTED (a head_dim
 *    or group size with no compiled kernel), PKV_EWORKSPACE (workspace too
 *    small).  PKV_EHIP reports a failed launch.  pkv_last_error() gives text.
 *  - Device-side values follow fixed rules instead of being checked:
 *      E = clamp(seqused_k[b], 0, min(max_seqlen_k, 16 * max_blocks_per_seq));
 *      column-mode kv_end below 0 counts as 0;
 *      row i of a unit with L query rows sits at position p = E - L + i and
 *      sees keys j with j < E, (causal: j <= p), (window > 0: j >= p - window + 1),
 *      (kv_start[u] = s > 0: j >= s, and a row with p < s sees only key p);
 *      a live key whose block-table entry is outside [0, num_blocks), or a
 *      segment whose column is outside [0, cols), contributes no keys;
 *      a row with no visible key is 0, and so is every row of [0, total_q)
 *      that no unit covers (rows of a unit past max_seqlen_q count as uncovered,
 *      so with max_seqlen_q = 1 each unit's row 0 alone is computed, at
 *      position E - L);
 *      only the live keys a unit can see are read: storage past seqused_k and
 *      block-table entries past ceil(E / 16) are never dereferenced, and
 *      values stored there (NaN included) never reach the output;
 *      a non-finite value in a key a row sees makes that row non-finite; a
 *      non-finite V value in a live key that another row of the same unit sees
 *      but this row does not (causal, window or kv_start rule) leaves this
 *      row's output unspecified (units of several rows multiply it by a zero
 *      weight in a dense product, and 0 * NaN is NaN); rows of other units and
 *      other kv heads are unaffected.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pkv_status {
    PKV_OK = 0,
    PKV_EINVAL = 1,
    PKV_EUNSUPPORTED = 2,
    PKV_EWORKSPACE = 3,
    PKV_EHIP = 4
} pkv_status;

typedef enum pkv_dtype {
    PKV_F32 = 0,
    PKV_BF16 = 1
} pkv_dtype;

#define PKV_BLOCK_SIZE 16

/*
 * pkv_kv_append -- write new K/V rows into slots of a flat cache view.
 * (vLLM-Omni paged_decode, PagedDecodeCache.attend: index_copy of this step's
 * K and V at the slot held in a device tensor; ExecuTorch PR #24073: in-graph
 * write to (position % rows) * columns + column.)
 *
 * k_cache, v_cache : [num_slots, kv_heads, head_dim], written in place.  A paged
 *                    cache [num_blocks, 16, kv_heads, head_dim] is the flat view
 *                    with num_slots = 16 * num_blocks; a column store
 *                    [rows, cols, kv_heads, head_dim] has num_slots = rows * cols.
 * k_new, v_new     : [num_tokens, kv_heads, head_dim], read only.
 * slot_mapping     : int64 [num_tokens]; token t goes to slot slot_mapping[t].
 *                    A slot outside [0, num_slots) is skipped.  Two tokens with
 *                    the same slot leave that slot undefined.
 * The copy moves raw 16/32-bit words: every bit pattern (NaN payloads included)
 * arrives unchanged.  num_tokens == 0 enqueues nothing and returns PKV_OK.
 */
pkv_status pkv_kv_append(void* k_cache, void* v_cache, int64_t num_slots,
                         const void* k_new, const void* v_new, int32_t num_tokens,
                         const int64_t* slot_mapping, int32_t kv_heads, int32_t head_dim,
                         pkv_dtype dtype, void* stream);

/*
 * pkv_paged_decode_attn -- one query token per sequence over a paged cache.
 * (vLLM-Omni paged_decode, PagedDecodeCache.attend with max_seqlen_q = 1,
 * cu_seqlens_q = [0, 1, ..], max_seqlen_k = bucket, causal = False.)
 *
 * out, q       : [num_seqs, q_heads, head_dim]; row b is sequence b's query.
 * k_cache, v_cache : [num_blocks, 16, kv_heads, head_dim].
 * block_table  : int32 [num_seqs, max_blocks_per_seq]; entry k names the pool
 *                block that holds tokens 16k .. 16k + 15 of the sequence.
 * seqused_k    : int32 [num_seqs], live keys per sequence, this step's included.
 * max_seqlen_k : host bound on seqused_k (the bucket).
 * k_new, v_new : optional [num_seqs, kv_heads, head_dim].  When both are given,
 *                the call first appends them at position seqused_k[b] - 1 of
 *                each sequence (the slot found through block_table; nothing for
 *                an empty sequence or an entry outside the pool) and then
 *                attends, as one step: inside the attention kernel on the
 *                vector path, as a launch of its own before the attention on
 *                the matrix-core path (bf16 with q_heads / kv_heads >= 8).
 *                When NULL the cache is only read.
 * softmax_scale: multiplies q.k before the softmax.
 * causal       : with one query per sequence causal equals non-causal.
 * window       : > 0 keeps the last `window` keys (p - window + 1 .. p).
 * kv_start     : optional int32 [num_seqs] left-padding bound (tiny-llm kv_cache.py,
 *                padded_causal_mask: first_valid per row): keys before
 *                kv_start[b] are hidden, and a query at a position before it (a
 *                pad query) sees only its own key.  NULL, or an entry <= 0, is no
 *                padding.  Keys below the bound never reach the output (NaN
 *                included), and whole 16-key blocks below it are not read.
 * num_splits   : split-K partitions per (sequence, kv head) on average; 0 lets the
 *                library pick from the host arguments.  With one sequence the
 *                live keys are cut into num_splits ranges; with several, the
 *                num_splits * num_seqs work groups of a kv head are dealt over the
 *                sequences by live length (on the device), so a long sequence
 *                takes more of them.  Results of different split counts agree to
 *                rounding; the same inputs and split count give the same bits.
 *                The library's own choice depends on the current device's
 *                compute-unit count.  On the matrix-core path (bf16, groups of
 *                8 and above) the num_splits * num_seqs work groups of a kv
 *                head are dealt the same way over the sequences.
 * workspace    : device scratch of at least pkv_attn_workspace_bytes(num_seqs, 1,
 *                max_seqlen_k, q_heads, kv_heads, head_dim, num_splits) bytes
 *                (may be NULL when that is 0).  It starts with split-K arrival
 *                counters, one 256-byte line per (sequence, kv head), that every
 *                call leaves at zero; the partials follow them.  Zero-fill it
 *                before its first use, and again before a call with another
 *                number of sequences or kv heads (or, for pkv_varlen_attn,
 *                another max_seqlen_q or head_dim) reuses it, since the counters
 *                then sit elsewhere; calls that differ only in lengths,
 *                num_splits or max_seqlen_k need no refill.  Calls that share a
 *                workspace must not run concurrently (one stream, or ordered
 *                streams).
 */
pkv_status pkv_paged_decode_attn(void* out, const void* q,
                                 const void* k_cache, const void* v_cache,
                                 int32_t num_blocks, int32_t block_size,
                                 const int32_t* block_table, int32_t max_blocks_per_seq,
                                 const int32_t* seqused_k, int32_t num_seqs, int32_t max_seqlen_k,
                                 const void* k_new, const void* v_new,
                                 int32_t q_heads, int32_t kv_heads, int32_t head_dim,
                                 float softmax_scale, int32_t causal, int32_t window,
                                 const int32_t* kv_start, int32_t num_splits, void* workspace,
                                 size_t workspace_bytes, pkv_dtype dtype, void* stream);

/*
 * pkv_varlen_attn -- packed query rows over a paged cache or a column store.
 * Exactly one of {block_table, seq_info} is non-NULL.
 *
 * out, q       : [total_q, q_heads, head_dim].
 * k, v         : paged mode [num_blocks, 16, kv_heads, head_dim];
 *                column mode [rows, cols, kv_heads, head_dim], key j of a
 *                segment in store row j % rows of its column.
 * Paged mode   : cu_seqlens_q int32 [num_seqs + 1] (sequence b owns rows
 *                cu_seqlens_q[b] .. cu_seqlens_q[b+1] - 1), seqused_k int32
 *                [num_seqs], block_table int32 [num_seqs, max_blocks_per_seq].
 * Column mode  : seq_info int32 [num_segments, 4] = (q_start, q_len, col, kv_end);
 *                num_segments <= 2 * cols.  Segments must not overlap in rows.
 *                With a window, rows must be >= window + max_seqlen_q - 1 (the
 *                ring then holds every key a step can see); without one, the
 *                caller keeps kv_end <= rows.
 * max_seqlen_q : host bound on any unit's query rows.
 * max_seqlen_k : host bound on the keys a unit sees.  Paged mode clamps
 *                seqused_k to it.  Column mode uses it only to choose the split
 *                count and requires it > 0 (e.g. window + max_seqlen_q - 1, or rows).
 * kv_start     : optional int32 [num_seqs] (paged) or [num_segments] (column):
 *                the left-padding bound of each unit, as for pkv_paged_decode_attn;
 *                with several query rows each row before the bound (a pad query)
 *                sees only its own key, causal or not.
 * Other arguments as for pkv_paged_decode_attn.  workspace must hold
 * pkv_attn_workspace_bytes(units, max_seqlen_q, ...) bytes with units =
 * num_seqs or num_segments.
 * Kernels: bf16 calls with max_seqlen_q = 1 and GQA groups below 8 run on the
 * vector path; bf16 calls that may hold units of several rows, or with groups
 * of 8 and above, on the matrix cores; fp32 takes every covered query row as a
 * single query on the vector path (fp32 products throughout), groups <= 8
 * only (PKV_EUNSUPPORTED above).
 */
pkv_status pkv_varlen_attn(void* out, const void* q, int32_t total_q,
                           const void* k, const void* v,
                           const int32_t* cu_seqlens_q, const int32_t* seqused_k, int32_t num_seqs,
                           const int32_t* block_table, int32_t max_blocks_per_seq,
                           int32_t num_blocks, int32_t block_size,
                           const int32_t* seq_info, int32_t num_segments, int32_t rows, int32_t cols,
                           int32_t max_seqlen_q, int32_t max_seqlen_k,
                           int32_t q_heads, int32_t kv_heads, int32_t head_dim,
                           float softmax_scale, int32_t causal, int32_t window,
                           const int32_t* kv_start, int32_t num_splits, void* workspace,
                           size_t workspace_bytes, pkv_dtype dtype, void* stream);

/*
 * pkv_prefix_import -- copy the first n positions of a dense prefill cache into
 * the paged cache and, optionally, set the live length to n.
 * (vLLM-Omni paged_decode, PagedDecodeCache.load_prefix and _write_prefix: the
 * [B, kv_heads, S, head_dim] prefill K/V of a layer, taken as one
 * [kv_heads, head_dim] row per position, written into the cache slots, then
 * set_length(prefix); from_dynamic_cache sizes the bucket for prefix + 1.)
 *
 * k_cache, v_cache : [num_blocks, 16, kv_heads, head_dim], written in place.
 * k_src, v_src     : [batch, kv_heads, src_len, head_dim], read only.
 * block_table      : int32 [batch, max_blocks_per_seq]; position j of sequence b
 *                    goes to slot 16 * block_table[b][j / 16] + j % 16.  A
 *                    position whose entry lies outside [0, num_blocks) is skipped;
 *                    entries past ceil(n / 16) are never read.
 * n                : positions copied per sequence; 0 <= n <= src_len and
 *                    n <= 16 * max_blocks_per_seq.
 * seqused_k        : optional int32 [batch]; when non-NULL every entry is set to n
 *                    by the same launch (set_length), so a following attention
 *                    call on the stream sees the imported prefix as live.
 * Raw 16/32-bit words are moved (NaN payloads arrive unchanged).  Slots not
 * written keep their contents: the tail past n is left as it was.  Two positions
 * whose tables name the same slot leave that slot undefined.  All four tensor
 * pointers must be 16-byte aligned (PKV_EINVAL otherwise).  batch == 0, or
 * n == 0 without seqused_k, enqueues nothing.
 */
pkv_status pkv_prefix_import(void* k_cache, void* v_cache, int32_t num_blocks, int32_t block_size,
                             const void* k_src, const void* v_src, int32_t batch, int32_t src_len,
                             int32_t n, const int32_t* block_table, int32_t max_blocks_per_seq,
                             int32_t* seqused_k, int32_t kv_heads, int32_t head_dim,
                             pkv_dtype dtype, void* stream);

/*
 * pkv_prefix_export -- copy the first n positions of each sequence out of the
 * paged cache into a dense cache.
 * (vLLM-Omni paged_decode, PagedDecodeCache.to_dynamic_cache: slots [:n] as a
 * contiguous [1, kv_heads, n, head_dim] for the stage that reads an ordinary
 * cache, once at hand-off.)
 *
 * k_dst, v_dst     : [batch, kv_heads, n, head_dim], every element written.
 * k_cache, v_cache : [num_blocks, 16, kv_heads, head_dim], read only.
 * block_table, n   : as for pkv_prefix_import (here src_len is n).  A position
 *                    whose entry lies outside [0, num_blocks) is written as zero
 *                    bits.
 * Raw words are moved; pointers must be 16-byte aligned.  batch == 0 or n == 0
 * enqueues nothing.
 */
pkv_status pkv_prefix_export(void* k_dst, void* v_dst, const void* k_cache, const void* v_cache,
                             int32_t num_blocks, int32_t block_size, int32_t batch, int32_t n,
                             const int32_t* block_table, int32_t max_blocks_per_seq,
                             int32_t kv_heads, int32_t head_dim, pkv_dtype dtype, void* stream);

/*
 * Batched-sequence column store: host bookkeeping (BatchControl).
 * (ExecuTorch PR #24073, the batched-sequence cache: one column per admitted
 * sequence of a [rows, max_seqs + 1, H, D] store, the last column scratch for
 * padded static-width writes; ring layers of min(capacity, window +
 * max_write - 1) rows; declare_step / prepare_step / commit_step, seq_clone,
 * seq_rm, rewind bounded by the ring floor, pos, max_seqs; one contiguous run
 * of tokens per owner in a step.  PR #24076: a ring grows like a flat store
 * until it first wraps, capped at its own rows.)
 *
 * The object lives on the host and touches no device memory: prepare_step
 * fills caller-owned host buffers that the caller uploads, and the device part
 * of a clone is pkv_column_copy.  A sequence id is its column.  Not thread-safe.
 *
 * pkv_batch_create : a ring store when window > 0 and window + max_write - 1 <=
 *                    capacity (rows = that sum, positions unbounded, slot of
 *                    position p in column c = (p % rows) * cols + c); otherwise
 *                    a flat store of `capacity` rows (a column is full at
 *                    capacity).  NULL on bad arguments (pkv_last_error says why).
 * pkv_batch_rows_needed : store rows a step of `step_width` tokens needs now,
 *                    rounded up to `row_step`, at most the store's rows (the
 *                    growth schedule of a flat store, or of a ring not yet
 *                    wrapped).
 * pkv_batch_seq_new : the lowest free column; PKV_EINVAL when all are taken.
 * pkv_batch_seq_clone : a new sequence at the source's position; *copy_rows
 *                    store rows of the source column hold its live keys and
 *                    must be copied (pkv_column_copy, every layer) before the
 *                    clone is used.
 * pkv_batch_rewind : move a sequence back to `pos`; PKV_EINVAL past its position
 *                    or below pkv_batch_floor (a ring must still hold the keys
 *                    a step starting at `pos` can see).
 * pkv_batch_declare_step : this step's owners in row order, n_tokens[i] in
 *                    1 .. max_write each, every owner at most once, their sum
 *                    <= width (the static token width of the step).
 * pkv_batch_prepare_step : seq_info [max_segments, 4] = (q_start, q_len, col,
 *                    kv_end = pos + q_len) per owner, zero rows after them; slots
 *                    int64 [width]: token t of an owner at position pos + t goes
 *                    to its column's slot, padding tokens to the scratch column.
 *                    Feed them to pkv_kv_append and pkv_varlen_attn (seq_info).
 * pkv_batch_commit_step : advances every owner by its tokens.
 * seq_new / seq_rm / seq_clone / rewind are refused between declare and commit.
 */
typedef struct pkv_batch pkv_batch;
pkv_batch* pkv_batch_create(int32_t max_seqs, int32_t capacity, int32_t window, int32_t max_write);
void pkv_batch_destroy(pkv_batch* b);
int32_t pkv_batch_max_seqs(const pkv_batch* b);
int32_t pkv_batch_cols(const pkv_batch* b);
int32_t pkv_batch_rows(const pkv_batch* b);
int32_t pkv_batch_rows_needed(const pkv_batch* b, int32_t step_width, int32_t row_step);
pkv_status pkv_batch_seq_new(pkv_batch* b, int32_t* seq);
pkv_status pkv_batch_seq_rm(pkv_batch* b, int32_t seq);
pkv_status pkv_batch_seq_clone(pkv_batch* b, int32_t src, int32_t* dst, int32_t* copy_rows);
pkv_status pkv_batch_rewind(pkv_batch* b, int32_t seq, int32_t pos);
pkv_status pkv_batch_pos(const pkv_batch* b, int32_t seq, int32_t* pos);
int32_t pkv_batch_floor(const pkv_batch* b, int32_t seq);
pkv_status pkv_batch_declare_step(pkv_batch* b, const int32_t* seqs, const int32_t* n_tokens,
                                  int32_t count, int32_t width);
pkv_status pkv_batch_prepare_step(pkv_batch* b, int32_t* seq_info, int32_t max_segments,
                                  int64_t* slots, int32_t* num_segments);
pkv_status pkv_batch_commit_step(pkv_batch* b);

/*
 * pkv_column_copy -- copy store rows [0, n_rows) of column src_col to column
 * dst_col in K and V (the device half of seq_clone).
 * k, v : [rows, cols, kv_heads, head_dim], 16-byte aligned.  Raw words move.
 * src_col == dst_col or n_rows == 0 enqueues nothing.
 */
pkv_status pkv_column_copy(void* k, void* v, int32_t rows, int32_t cols, int32_t kv_heads,
                           int32_t head_dim, int32_t src_col, int32_t dst_col, int32_t n_rows,
                           pkv_dtype dtype, void* stream);

/*
 * pkv_paged_decode_attn_noalloc -- pkv_paged_decode_attn for callers that cannot
 * allocate device memory: code under hipGraph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, meaning and results as
 * pkv_paged_decode_attn, without the workspace.
 *
 * Its split-K scratch is a static device array of PKV_NOALLOC_SCRATCH_BYTES
 * that the library holds on every GPU it runs on until the process ends; the
 * call allocates and frees nothing.
 *  - A call whose arguments need more scratch than that
 *    (pkv_attn_workspace_bytes with the same arguments) returns PKV_EWORKSPACE
 *    before enqueuing anything: pass a smaller num_splits, or use
 *    pkv_paged_decode_attn with a caller workspace.
 *  - Each call first clears the scratch's split-K arrival counters with a
 *    small kernel on `stream` (the array keeps the previous call's contents),
 *    then enqueues the attention as pkv_paged_decode_attn does.
 *  - Every call on one GPU uses the same array: calls that overlap in time on
 *    one GPU (other streams, other host threads) race and give undefined
 *    results.  Order them, e.g. on one stream.
 *  - The first call on a device looks up the array's address there
 *    (hipGetSymbolAddress); make that first call outside stream capture.
 */
#define PKV_NOALLOC_SCRATCH_BYTES (16u << 20)
pkv_status pkv_paged_decode_attn_noalloc(void* out, const void* q,
                                         const void* k_cache, const void* v_cache,
                                         int32_t num_blocks, int32_t block_size,
                                         const int32_t* block_table, int32_t max_blocks_per_seq,
                                         const int32_t* seqused_k, int32_t num_seqs,
                                         int32_t max_seqlen_k, const void* k_new, const void* v_new,
                                         int32_t q_heads, int32_t kv_heads, int32_t head_dim,
                                         float softmax_scale, int32_t causal, int32_t window,
                                         const int32_t* kv_start, int32_t num_splits,
                                         pkv_dtype dtype, void* stream);

/*
 * pkv_attn_workspace_bytes -- device scratch an attention call with these host
 * arguments needs (split-K partials); 0 when it needs none.  `units` is num_seqs
 * (paged) or num_segments (column); num_splits as passed to the call.  With
 * num_splits = 0 the answer depends on the current device (its compute-unit
 * count), so ask with the device current that will run the call.  The size
 * covers bf16 and fp32 calls alike.
 */
size_t pkv_attn_workspace_bytes(int32_t units, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                int32_t q_heads, int32_t kv_heads, int32_t head_dim,
                                int32_t num_splits);

/* Split count the library uses for a bf16 call with these host arguments
 * (num_splits = 0 picks): the vector path's for calls of single-row units with
 * groups below 8, else the matrix-core path's. */
int32_t pkv_attn_num_splits(int32_t units, int32_t max_seqlen_q, int32_t max_seqlen_k,
                            int32_t q_heads, int32_t kv_heads, int32_t head_dim,
                            int32_t num_splits);

/* Static text for a status code. */
const char* pkv_status_string(pkv_status s);

/* Detail of the last non-OK return on the calling thread ("" if none). */
const char* pkv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
