/*
 * cpattn.h -- C ABI of libcpattn.so: one context-parallel rank's share of
 * zigzag prefill attention on AMD Instinct MI355X (gfx950), plus the host
 * metadata, the KV-pool scatter and the zigzag rerange around it, and the
 * non-causal AllGather-KV (local Q / global K/V) variant.
 *
 * Sources (web pages; cited by title and section):
 *   [P1] "Zigzag cp #3" pull request page (alexsun07/sglang): prefill CP on
 *        ROCm gathers K/V into the local pool, then runs the prev and next
 *        zigzag halves; lengths come from host metadata, no host sync, and a
 *        preallocated kv_indptr instead of per-call tensors.
 *   [P2] vllm-omni pull request #7937 "Compose Ulysses with AllGather-KV as a
 *        2D SP topology": local Q against global K/V; the K/V pad is a strict
 *        suffix that no query consumes; unsupported combinations fail closed;
 *        query offsets must be local row indices.
 *   [P4] prhub report on sglang pull request #34485 (AITer backend takes
 *        grouped-query K/V): num_heads must be a multiple of num_kv_heads,
 *        each KV head serves a contiguous group of query heads, the softmax
 *        scale is head_size ** -0.5.
 *   [P5] sglang source page python/sglang/srt/layers/cp/zigzag.py: module
 *        docstring (block layout), ZigzagContextParallelMetadata,
 *        ZigzagCPStrategy.can_apply / build_metadata / shard_hidden_states /
 *        gather_kv_cache / run_attention / materialize_full_kv /
 *        _all_gather_reorganized.
 *
 * Conventions shared by every entry point
 *   - Return 0 (CP_OK) on success or a negative cp_status_t.  Nothing throws.
 *   - Every argument is validated on the host BEFORE anything is enqueued; on
 *     error nothing is written and nothing is launched (fail closed, [P2]).
 *     cp_last_error() returns a thread-local message naming the argument.
 *   - No call allocates device memory, copies device->host, or synchronises
 *     a stream or the device ([P1]).  Device work is enqueued on the caller's
 *     stream; the caller owns every buffer and every stream.
 *   - Tensors are token-major: [rows, heads, D] with D innermost, bf16.
 *   - Device pointers passed to the copy and attention calls must be 16-byte
 *     aligned; source and destination buffers must not overlap.
 */
#ifndef CPATTN_H_
#define CPATTN_H_

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum cp_status {
  CP_OK = 0,
  CP_ERR_INVALID_ARG = -1,      /* an argument is out of its documented range */
  CP_ERR_UNSUPPORTED = -2,      /* well-formed but not supported (e.g. D not 64/128) */
  CP_ERR_BUFFER_TOO_SMALL = -3, /* a caller buffer is smaller than required */
  CP_ERR_OVERFLOW = -4,         /* a count or offset does not fit the index width */
  CP_ERR_HIP = -5               /* the HIP runtime reported an error at launch */
} cp_status_t;

enum { CP_META_VERSION = 3 };
enum { CP_META_ZIGZAG = 1, CP_META_ALLGATHER = 2 };
enum { CP_RERANGE_GATHERED_TO_ORIG = 0, CP_RERANGE_ORIG_TO_GATHERED = 1 };

/*
 * Host summary of one metadata blob.
 *
 * The blob is one caller-owned host buffer holding every int32 array below
 * at the listed byte offsets (each offset is a multiple of 256).  The caller
 * reads the lists from the host copy and copies the whole blob (blob_bytes)
 * to a device buffer with hipMemcpyAsync on its stream; the copy and
 * attention calls take that device copy (d_blob) plus this struct.  The copy
 * calls only read d_blob.  cp_prefill_attn also updates a 36-byte job-counter
 * area in its 256-byte header while it runs and leaves it as the builder
 * wrote it (zero), so two attention launches that share one d_blob must not
 * run at the same time: order them on one stream, or give each its own copy.
 *
 * Lists of [P5] ZigzagContextParallelMetadata (int32):
 *   split_list[bs*2cp]         block sizes, sequence-major
 *   zigzag_index[2*bs]         chunk ids this rank keeps: early blocks of all
 *                              sequences, then late blocks
 *   cp_reverse_index[bs*2cp]   for each original chunk, its chunk position in
 *                              the all-gathered (rank-major) buffer
 *   reverse_split_len[bs*2cp]  chunk sizes of the all-gathered buffer
 *   per_rank_actual_token[cp]  real rows each rank contributes
 *   kv_len_prev[bs], kv_len_next[bs]       keys seen by each half (incl. prefix)
 *   q_prev[bs], q_next[bs]                 query rows of each half
 *   cu_seqlens_q_prev[bs+1], cu_seqlens_q_next[bs+1]
 *   prefix[bs], extend[bs]     cached prefix and extend length per sequence
 * Tables of this library (opaque layout, used by the kernels):
 *   chunks, segments, work list.
 */
typedef struct cp_meta {
  int32_t version;            /* CP_META_VERSION */
  int32_t kind;               /* CP_META_ZIGZAG (causal) or CP_META_ALLGATHER */
  int32_t cp_size, cp_rank, bs;  /* bs: sequences = rows of the page table the attention reads (1 for AllGather-KV) */
  int32_t attn_group;         /* H_q/H_kv the work list was built for; 0 = none */
  int64_t total_seq_lens;     /* sum of extend lengths (after any surplus) */
  int32_t max_rank_len;       /* rows per rank in the all-gathered buffer */
  int32_t total_q_prev_tokens, total_q_next_tokens;
  int32_t max_seqlen_q_prev, max_seqlen_q_next;
  int32_t n_local_rows;       /* this rank's Q/O rows */
  int32_t n_chunks;           /* bs*2cp (zigzag), 0 (allgather) */
  int32_t max_chunk_rows;
  int32_t n_seg;              /* attention segments: 2*bs (zigzag), 1 or one per document (allgather) */
  int32_t n_work;             /* attention work items */
  int32_t max_kv_len;
  int32_t q_tile;             /* query positions per work item */
  int32_t kv_align;           /* largest power of two (<= 2^30) dividing every segment's first key
                                 position in its page-table row (2^30 when all start at 0) */
  int32_t mean_item_tiles;    /* mean 64-key tiles per work item, rounded down (0: no items) */
  int64_t blob_bytes;         /* bytes of the blob that are in use */
  int64_t off_split_list, off_zigzag_index, off_cp_reverse_index, off_reverse_split_len;
  int64_t off_per_rank_actual_token, off_kv_len_prev, off_kv_len_next;
  int64_t off_q_prev, off_q_next, off_cu_seqlens_q_prev, off_cu_seqlens_q_next;
  int64_t off_prefix, off_extend;
  int64_t off_chunks, off_segs, off_work;
} cp_meta_t;

/*
 * cp_meta_build -- host-only zigzag metadata of rank cp_rank ([P5]
 * build_metadata, validity from can_apply).
 *
 *   extend_lens[bs]  required: new tokens per sequence.
 *   seq_lens[bs]     nullable: full lengths; prefix_b = max(seq_b - extend_b, 0)
 *                    tokens are already cached ahead of the extend part.
 *   num_tokens       rows of the batch; any surplus over sum(extend_lens) is
 *                    added to the last sequence (and to its seq_len).
 *   attn_group       H_q/H_kv for the attention work list (0: no list;
 *                    cp_prefill_attn then rejects this metadata).
 *   blob, blob_capacity  caller-owned host buffer.  With blob == NULL the call
 *                    only fills *meta (meta->blob_bytes is the size to
 *                    allocate) and returns CP_OK.
 * Errors: cp_size < 2, cp_rank outside [0, cp_size), bs < 1, any extend
 * length < 2*cp_size, num_tokens < sum(extend_lens) -> CP_ERR_INVALID_ARG
 * (can_apply is false); attn_group outside [0, 256] -> CP_ERR_UNSUPPORTED;
 * totals >= 2^31 -> CP_ERR_OVERFLOW; blob_capacity < blob_bytes ->
 * CP_ERR_BUFFER_TOO_SMALL.  Pure host code: no HIP call.
 */
int cp_meta_build(int32_t cp_size, int32_t cp_rank, int32_t bs,
                  const int32_t* extend_lens, const int32_t* seq_lens,
                  int64_t num_tokens, int32_t attn_group,
                  void* blob, int64_t blob_capacity, cp_meta_t* meta);

/*
 * cp_allgather_meta_build -- host-only metadata of the non-causal
 * AllGather-KV share ([P2]): q_total local query rows, of which the first
 * q_real are real, attend to keys [0, kv_len) of the ordered global K/V; the
 * K/V rows at and past kv_len (the pad suffix) are never read, and output
 * rows at and past q_real are written as zeros.  Query rows are local
 * indices ([P2] review of the packed offsets).
 * Errors: q_total < 1, q_real outside [0, q_total], kv_len < 1 ->
 * CP_ERR_INVALID_ARG; attn_group outside [1, 256] -> CP_ERR_UNSUPPORTED.
 * Blob handling as in cp_meta_build.
 */
int cp_allgather_meta_build(int32_t q_total, int32_t q_real, int32_t kv_len,
                            int32_t attn_group, void* blob, int64_t blob_capacity,
                            cp_meta_t* meta);

/*
 * cp_allgather_packed_meta_build -- host-only metadata of the non-causal
 * AllGather-KV share when the global sequence packs several documents
 * ([P2]: the query ranges of a rank's local slice and the local query
 * boundaries remapped from the global ones).
 *   doc_cu[n_docs+1]: document boundaries in the global sequence, exclusive
 *     prefix sums of the real lengths (doc_cu[0] = 0, non-decreasing);
 *     global rows at and past doc_cu[n_docs] are the pad suffix.
 *   The local query rows are global rows [q_start, q_start + q_total).  A
 *   local row of document b attends, with no causal mask, to K/V rows
 *   doc_cu[b] .. doc_cu[b+1]-1 of the ordered global K/V (page-table row 0);
 *   rows in the pad suffix are written as zeros and pad K/V rows are never
 *   read.  One segment per document that meets the slice.
 * The Ulysses head share is a plain smaller head count at the attention
 * call (H_q/U query heads, their KV heads).
 * Errors: n_docs < 1, NULL doc_cu, doc_cu[0] != 0, decreasing doc_cu, no real
 * row, q_total < 1, q_start < 0 -> CP_ERR_INVALID_ARG; q_start + q_total
 * beyond int32 -> CP_ERR_OVERFLOW; attn_group outside [1, 256] ->
 * CP_ERR_UNSUPPORTED.  Blob handling as in cp_meta_build.
 */
int cp_allgather_packed_meta_build(int32_t n_docs, const int32_t* doc_cu, int32_t q_start,
                                   int32_t q_total, int32_t attn_group, void* blob,
                                   int64_t blob_capacity, cp_meta_t* meta);

/*
 * cp_zigzag_rerange -- bit copy of whole rows between the all-gathered
 * layout and original token order ([P5] gather_kv_cache /
 * gather_hidden_states after _all_gather_reorganized, and shard_* for every
 * rank at once).
 *   CP_RERANGE_GATHERED_TO_ORIG: src [cp*max_rank_len, row] -> dst
 *     [total_seq_lens, row]; each rank's pad rows are skipped.
 *   CP_RERANGE_ORIG_TO_GATHERED: src [total_seq_lens, row] -> dst
 *     [cp*max_rank_len, row]; every rank's shard lands at its slot, pad rows
 *     of dst are left untouched.
 *   row_bytes: any positive row size.  Multiples of 16 (K/V rows, hidden
 *   states) move as 16-byte vectors; other sizes (int32/int64 positions,
 *   narrow per-token tensors) in elements of the widest power of two up to
 *   8 bytes that divides row_bytes.  src and dst must be 16-byte aligned and
 *   must not overlap.
 * Errors: NULL meta or d_blob, meta kind not zigzag (or another version), bad
 * direction, row_bytes <= 0, NULL or misaligned pointers -> CP_ERR_INVALID_ARG;
 * a grid of more than 2^24-1 workgroups (16 KiB each: HIP's 2^32-1 work-item
 * limit at 256 threads) -> CP_ERR_OVERFLOW; launch failure -> CP_ERR_HIP.
 */
int cp_zigzag_rerange(const void* d_blob, const cp_meta_t* meta, int32_t direction,
                      const void* src, void* dst, int64_t row_bytes, hipStream_t stream);

/*
 * cp_zigzag_rerange_kv -- cp_zigzag_rerange of K and of V in one launch
 * (gather_kv_cache reranges both after the all-gather, [P5]).  Arguments,
 * layout, ownership and errors are those of cp_zigzag_rerange, applied to
 * each of the pairs (k_src -> k_dst) and (v_src -> v_dst), which share
 * row_bytes; the result is bit-identical to the two separate calls.  Rows
 * whose size is not a multiple of 16 bytes are copied by those two calls.
 */
int cp_zigzag_rerange_kv(const void* d_blob, const cp_meta_t* meta, int32_t direction,
                         const void* k_src, void* k_dst, const void* v_src, void* v_dst,
                         int64_t row_bytes, hipStream_t stream);

/*
 * cp_kv_scatter -- gathered K and V rows into the paged KV pool ([P5]
 * materialize_full_kv: gather, rerange, write at the extend tokens' cache
 * locations; [P1]: every rank's pool then holds the full sequence).
 *   k_gathered, v_gathered: [cp*max_rank_len, H_kv, D] bf16, rank-major with
 *     pad rows (never read).
 *   k_pool, v_pool: [num_pages, page_size, H_kv, D] bf16.
 *   kv_page_indptr[bs+1], kv_page_indices[...]: int32 device arrays (CSR);
 *     page j of sequence b is kv_page_indices[kv_page_indptr[b] + j].
 *   Extend token t of sequence b goes to sequence position prefix_b + t, i.e.
 *   page (prefix_b+t)/page_size, slot (prefix_b+t)%page_size.  No other slot
 *   is written.  The page table is read only on the device, and only inside
 *   each sequence's row: entry j of sequence b is read only when
 *   j < kv_page_indptr[b+1] - kv_page_indptr[b].  A token whose entry lies
 *   past its row, or whose page id falls outside [0, num_pages), is skipped
 *   (its slot is not written; nothing is written out of bounds).  The CSR
 *   itself (indptr non-decreasing, kv_page_indices holding indptr[bs]
 *   entries) is the caller's contract.
 * Errors: NULL meta or d_blob, meta kind not zigzag (or another version),
 * H_kv < 1, D < 1, page_size < 1, num_pages < 1, NULL or misaligned pointers
 * -> CP_ERR_INVALID_ARG; H_kv*D*2 not a multiple of 16 -> CP_ERR_UNSUPPORTED;
 * a grid of more than 2^24-1 workgroups (one per 2 KiB of a page run of a
 * chunk: HIP's 2^32-1 work-item limit at 256 threads) -> CP_ERR_OVERFLOW;
 * launch failure -> CP_ERR_HIP.
 */
int cp_kv_scatter(const void* d_blob, const cp_meta_t* meta,
                  const void* k_gathered, const void* v_gathered,
                  void* k_pool, void* v_pool, int32_t num_pages, int32_t page_size,
                  int32_t H_kv, int32_t D,
                  const int32_t* kv_page_indptr, const int32_t* kv_page_indices,
                  hipStream_t stream);

/*
 * cp_prefill_attn -- one fused launch over every segment of the metadata:
 * both zigzag halves of every sequence (CP_META_ZIGZAG, causal) or the
 * AllGather-KV segments, one per document of the local slice
 * (CP_META_ALLGATHER, non-causal) ([P5] run_attention, [P1], [P2]).
 *   For segment (half, b) with q_len rows starting at local row r0 and
 *   kv_len keys: O[r0+i, h] = softmax(scale * Q[r0+i, h] K^T + M) V over keys
 *   0..kv_len-1 of sequence b, read through the page table; KV head of query
 *   head h is h / (H_q/H_kv) ([P4]); causal M hides key j > i + kv_len - q_len
 *   (bottom-right alignment).
 *   q, out: [n_local_rows, H_q, D] bf16, local order (prev halves of all
 *     sequences, then next halves).  Fp32 accumulation, bf16 output (RNE).
 *   k_pool, v_pool, num_pages, page table: as in cp_kv_scatter.  A
 *     contiguous [S, H_kv, D] tensor is the pool with page_size dividing S
 *     and the identity page table.  Page-table reads stay inside the
 *     segment's row: a row with fewer than ceil(keys / page_size) entries
 *     repeats its last entry for the missing ones, and an empty row reads as
 *     an invalid page id.  A key whose page id lies outside [0, num_pages)
 *     is read from the first slot of the segment's page-table row instead
 *     (or slot 0 of the pool).  Neither case reads out of bounds, but such a
 *     table gives unspecified results.
 *   meta->kv_align picks how page ids are fetched for pages under 64 keys
 *     (whole pages per key tile when it is >= page_size); a meta whose
 *     kv_align overstates the segments' alignment gives unspecified results,
 *     again with no out-of-bounds read.  The meta builders set it exactly.
 *   Scheduling: one workgroup per job (work item, KV head).  When there are
 *     more jobs than compute units and items average at least 48 key tiles
 *     (meta->mean_item_tiles), the first round of jobs (one per compute unit)
 *     is fixed and the rest are handed out at run time from 8 queues, one per
 *     XCD, from which an XCD whose own queue is empty takes the next job of
 *     another's; the grid then holds up to 1/8 more workgroups, which find no
 *     job and end at once.  The job counters live in d_blob's header (see the
 *     blob description above): launches that share a blob must not overlap.
 *     A job's result does not depend on where it runs: outputs are
 *     bit-identical from launch to launch.
 * Errors: NULL meta or d_blob, unknown meta kind or version, H_q % H_kv != 0
 * ([P4]), H_q/H_kv different from meta->attn_group (the work list's), scale
 * not finite or <= 0, num_pages < 1, NULL or misaligned (16-byte) pointers
 * -> CP_ERR_INVALID_ARG; D not in {64, 128}, H_kv*D*2*64 >= 2^31 (one 64-key
 * tile of all KV heads), page_size not a power of two up to 2^20 ->
 * CP_ERR_UNSUPPORTED; a grid (n_work * H_kv workgroups of 512 threads, plus
 * the spare ones of run-time scheduling) of more than 2^23-1 workgroups
 * (HIP's 2^32-1 work-item limit) -> CP_ERR_OVERFLOW; a failing query of the
 * device's compute-unit count or a launch failure -> CP_ERR_HIP.
 */
int cp_prefill_attn(const void* q, const void* k_pool, const void* v_pool, void* out,
                    int32_t H_q, int32_t H_kv, int32_t D, float scale,
                    void* d_blob, const cp_meta_t* meta,
                    int32_t num_pages, int32_t page_size, const int32_t* kv_page_indptr,
                    const int32_t* kv_page_indices, hipStream_t stream);

/*
 * cp_prefill_attn_noalloc -- for callers that cannot allocate device memory
 * for a launch's working state or must not have their metadata written (code
 * under HIP graph capture that treats the blob as read-only, tight serving
 * loops, harnesses that forbid allocation).  Same arguments, computation,
 * results (bit for bit) and errors as cp_prefill_attn, but d_blob is only
 * read: the run-time job counters live in a file-scope device array of the
 * library (9 words, 36 bytes, fixed: no input size needs more; each GPU holds
 * its own copy until the process ends).  Its device address is looked up
 * once per device (hipGetSymbolAddress, with that device current); nothing
 * is allocated, here or later.  Every launch leaves the counters zero, the
 * state the next launch needs.  All calls on one GPU share the array, so
 * calls that overlap in time on one GPU race and give wrong results: order
 * them on one stream.
 * Extra errors: the stream belonging to a device other than the current one
 * -> CP_ERR_INVALID_ARG; a failing symbol lookup -> CP_ERR_HIP.
 */
int cp_prefill_attn_noalloc(const void* q, const void* k_pool, const void* v_pool, void* out,
                            int32_t H_q, int32_t H_kv, int32_t D, float scale,
                            const void* d_blob, const cp_meta_t* meta,
                            int32_t num_pages, int32_t page_size, const int32_t* kv_page_indptr,
                            const int32_t* kv_page_indices, hipStream_t stream);

/* Thread-local description of the last error of this thread ("" if none). */
const char* cp_last_error(void);

/* Library version string. */
const char* cp_version(void);

#ifdef __cplusplus
}
#endif
#endif /* CPATTN_H_ */
