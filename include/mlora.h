/*
 * mlora.h — C ABI of the dynamic multi-LoRA library for MI355X (gfx950).
 *
 * What it computes (the pages, by title and section):
 *   - "vLLM-Ascend dynamic LoRA operator" walkthrough (pwwt.cn):
 *       s1.1  A is [r, K], B is [N, r]; y = y_base + (x A^T) B^T per token;
 *       s2.1  one lora id per token, -1 = none; weights packed by rank group
 *             and found through a per-id offset table;
 *       s2.2  two serial products, S = x A^T then S B^T, S accumulated in fp32;
 *       s2.3  tokens clustered by id into a segment table; one launch serves
 *             every segment;
 *       s3.4  a -1 token's base row passes through untouched;
 *       s4.3  ranks padded to a multiple of 16 with zero A rows / B columns;
 *             an all -1 batch launches nothing.
 *   - SGLang "LoRA Layers" page: shrink (lora_A) / expand (lora_B) calls,
 *     stacked QKV A (3r, in) / B (q+2kv, r) and gate-up A (2r, in) /
 *     B (2*out, r), the expand's output offsets, the rank-0 no-op slot.
 *   - SGLang "LoRA + MoE" page: LoRAInfo stacks, per (adapter, expert)
 *     alignment padded to block_size_m, gate/up delta before silu_and_mul,
 *     down delta before the top-k reduce, adapter_enabled mask.
 *
 * Conventions for every entry point:
 *   - Pointers named *device* are HIP device pointers; everything else is
 *     host memory that is read during the call only.
 *   - Every launch goes on `stream` in stream order.  No entry point
 *     synchronises the host, allocates or frees memory, or keeps a pointer
 *     after its work on the stream has finished (except
 *     lora_read_device_error, which synchronises `stream`).
 *   - The caller owns every buffer.  y / cache1 / cache3 are updated in
 *     place.  Weights must not change while work that reads them is queued.
 *   - Arguments are checked before any launch; a bad argument returns
 *     LORA_INVALID_ARG (or LORA_UNSUPPORTED for a valid but unsupported
 *     shape) and launches nothing.  A failed launch returns LORA_HIP_ERROR.
 *   - Dtypes: x, A, B and y share one dtype (LORA_BF16 or LORA_F32); S,
 *     routing weights and all accumulation are fp32; results are rounded to
 *     the storage dtype once (round to nearest even).
 *   - Device pointers to x / y / A / B / cache buffers must be 16-byte
 *     aligned; leading dimensions and K, N are multiples of 8 elements.
 *   - Profiling: with the environment variable MLORA_ROCTX=1 set before the
 *     first call, every entry point that launches work (and
 *     lora_read_device_error) is bracketed by a roctx range named after it
 *     (rocprofv3 --marker-trace shows them).  The roctx library is looked up
 *     at run time; without it, or without the variable, no range is made.
 */
#ifndef MLORA_H
#define MLORA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLORA_ABI_VERSION 5

typedef enum lora_status {
    LORA_OK = 0,
    LORA_INVALID_ARG = 1,
    LORA_UNSUPPORTED = 2,
    LORA_HIP_ERROR = 3
} lora_status;

typedef enum lora_dtype {
    LORA_F32 = 0,
    LORA_BF16 = 1
} lora_dtype;

#define LORA_MAX_SLICES 4      /* stacked output slices per call (QKV = 3, gate-up = 2) */
#define LORA_RANK_ALIGN 16     /* ranks are padded to a multiple of this */
#define LORA_MAX_RANK 64       /* padded rank per slice */
#define LORA_MAX_ADAPTERS 1024 /* adapter slots per table */
#define LORA_DECODE_MAX_M 64   /* token count up to which the fused decode kernel runs */

/*
 * Packed weight table (Ascend walkthrough s2.1 and s4.3; SGLang "LoRA Layers"
 * stacked shapes).  Adapter i with padded rank rp = rank[i] owns
 *   A rows  A + a_off[i] : [n_slices * rp, K] row-major; rows [s*rp, (s+1)*rp)
 *                          belong to slice s, rows past the true rank are 0;
 *   B rows  B + b_off[i] : [N_total, rp] row-major; rows
 *                          [slice_offsets[s], slice_offsets[s+1]) belong to
 *                          slice s, columns past the true rank are 0.
 * rank[i] == 0 marks an empty (no-op) slot.  Offsets are in elements.
 */
typedef struct lora_weights {
    int32_t dtype;              /* lora_dtype */
    int32_t K;                  /* input width */
    int32_t n_slices;           /* 1..LORA_MAX_SLICES */
    int32_t L;                  /* adapter slots */
    int32_t r_max;              /* max of rank[] (multiple of 16, <= 64) */
    int32_t reserved;
    int64_t slice_offsets[LORA_MAX_SLICES + 1]; /* host values; [0] == 0, increasing, [n_slices] = N_total */
    const void* A;              /* device: packed A table */
    const void* B;              /* device: packed B table */
    const int64_t* a_off;       /* device [L] */
    const int64_t* b_off;       /* device [L] */
    const int32_t* rank;        /* device [L]: padded rank, 0 = empty slot */
} lora_weights_t;

/*
 * Segment table (Ascend walkthrough s2.3), built on the device by
 * lora_build_segments; counts never travel to the host.
 *   sorted_idx   [M]   tokens ordered by ascending adapter id, stable; tokens
 *                      without an adapter come last and are in no segment;
 *   seg_indptr   [L+1] segment s covers sorted positions [seg_indptr[s], seg_indptr[s+1]);
 *                      entries past num_segments equal the number of tokens with an adapter;
 *   req_to_lora  [L]   adapter id of segment s; -1 past num_segments;
 *   num_segments [1]   number of non-empty segments.
 * Tile schedule (walkthrough s2.4: block -> segment -> rank settled before
 * the product kernels run): each segment is cut into tiles of
 * LORA_TILE_ROWS sorted positions.
 *   tile_info    [max_tiles][4]  segment, adapter id, first sorted position, rows;
 *   tile_rows    [max_tiles][LORA_TILE_ROWS] token index of each row, -1 past the rows;
 *   num_tiles    [1]   number of tiles;
 *   max_tiles    capacity, >= lora_tile_capacity(M, L).
 */
#define LORA_TILE_ROWS 64

typedef struct lora_segments {
    const int32_t* sorted_idx;   /* device */
    const int32_t* seg_indptr;   /* device */
    const int32_t* req_to_lora;  /* device */
    const int32_t* num_segments; /* device */
    const int32_t* tile_info;    /* device */
    const int32_t* tile_rows;    /* device */
    const int32_t* num_tiles;    /* device */
    int32_t L;                   /* capacity the table was built with (== weights L) */
    int32_t max_tiles;           /* tile capacity the table was built with */
} lora_segments_t;

/* ---------------------------------------------------------------- common */

/* Library ABI version (MLORA_ABI_VERSION). */
int32_t lora_abi_version(void);

/* Static description of a status code; never NULL. */
const char* lora_status_string(lora_status status);

/*
 * Bytes of device workspace needed by lora_shrink / lora_shrink_expand_add
 * for this table and up to M tokens.  The workspace must be zeroed once
 * (lora_workspace_init) before its first use; the kernels leave it ready for
 * the next call.  Calls that share a workspace must be ordered on one stream.
 */
size_t lora_workspace_size(const lora_weights_t* w, int32_t M);

/* Zero `bytes` of device workspace with a fill kernel on `stream`. */
lora_status lora_workspace_init(void* workspace, size_t bytes, hipStream_t stream);

/*
 * Read (and clear) the sticky device error word of a workspace.  Synchronises
 * `stream`.  *out receives 0 when no kernel reported an error, else an OR of
 *   LORA_DEVERR_WAIT    a kernel gave up waiting on data from another
 *                       workgroup; the results of that call are not valid
 *                       (the workspace itself stays usable).  A library
 *                       built with MLORA_DEBUG and run with
 *                       MLORA_DEBUG_WAIT_FAULT=1 in the environment makes
 *                       every such wait give up after a few polls, to test
 *                       this path;
 *   LORA_DEVERR_BAD_ID  lora_fused_decode met a token id outside [-1, L); the
 *                       token was treated as one without an adapter.  An id
 *                       past the table would index a slot that does not
 *                       exist, the mixed-up-rows failure of the Ascend
 *                       walkthrough's s4.1 troubleshooting table, so it is
 *                       reported and never followed.
 *   LORA_DEVERR_TABLE   (libraries built with MLORA_DEBUG only) a
 *                       table-form call met a segment-table entry that does
 *                       not fit the batch or the weight table: an adapter
 *                       id outside [0, L), a token index outside [0, M), or
 *                       a tile or segment reaching past M.  The tile or
 *                       segment is skipped, never dereferenced.  Calls
 *                       without a workspace (lora_expand_add,
 *                       lora_embedding_shrink) skip such entries without
 *                       reporting them.  The release library does not check.
 */
#define LORA_DEVERR_WAIT 1
#define LORA_DEVERR_BAD_ID 2
#define LORA_DEVERR_TABLE 4

lora_status lora_read_device_error(void* workspace, int32_t* out, hipStream_t stream);

/* ---------------------------------------------------------------- weight table (load time) */

/*
 * Plan a packed table (Ascend walkthrough s2.1: weights grouped by rank so
 * that each rank group is contiguous; s4.3: rank padded to 16).
 *   ranks     host [L]  true ranks (0 = empty slot), each <= LORA_MAX_RANK;
 *   rank_pad  host [L]  out: padded ranks;
 *   a_off, b_off host [L] out: element offsets (rank-group major, then slot);
 *   a_elems, b_elems    out: total elements of the A and B tables.
 * Host only; launches nothing.
 */
lora_status lora_table_plan(int32_t L, const int32_t* ranks, int32_t n_slices, int32_t K,
                            int64_t N_total, int32_t* rank_pad, int64_t* a_off, int64_t* b_off,
                            int64_t* a_elems, int64_t* b_elems);

/*
 * Copy one adapter into its slot of a packed table, writing the zero padding.
 *   A_src device [n_slices*rank, K] row-major (slice s = rows [s*rank, (s+1)*rank));
 *   B_src device [N_total, rank] row-major;
 *   A_dst device: table A + a_off[i]; B_dst device: table B + b_off[i].
 * rank_pad must be rank rounded up to 16.  rank == 0 writes nothing.
 */
lora_status lora_pack_adapter(int32_t dtype, int32_t K, int64_t N_total, int32_t n_slices,
                              int32_t rank, int32_t rank_pad, const void* A_src,
                              const void* B_src, void* A_dst, void* B_dst, hipStream_t stream);

/* ---------------------------------------------------------------- dense multi-LoRA */

/* Tile capacity for M tokens and L slots: floor(M / LORA_TILE_ROWS) + min(L, M). */
int32_t lora_tile_capacity(int32_t M, int32_t L);

/*
 * lora_build_segments (Ascend walkthrough s2.3; one workgroup, stable
 * counting sort on the device) and the tile schedule.
 *   ids device [M] int32: adapter id per token; -1 (or any id outside
 *       [0, L)) means no adapter.
 *   adapter_enabled device [L] int32, or NULL (every adapter enabled): a
 *       token whose adapter has adapter_enabled == 0 is treated like a
 *       token without an adapter (SGLang "LoRA + MoE" page: the per-adapter
 *       enable mask that lets one captured graph serve any active set).
 *   outputs device: sorted_idx [M], seg_indptr [L+1], req_to_lora [L],
 *       num_segments [1], tile_info [max_tiles][4],
 *       tile_rows [max_tiles][LORA_TILE_ROWS], num_tiles [1], as described
 *       for lora_segments_t.
 * 0 <= M <= 2^24, 1 <= L <= LORA_MAX_ADAPTERS,
 * max_tiles >= lora_tile_capacity(M, L).  M == 0 still writes the (empty)
 * table.
 */
lora_status lora_build_segments(const int32_t* ids, const int32_t* adapter_enabled, int32_t M,
                                int32_t L, int32_t* sorted_idx, int32_t* seg_indptr,
                                int32_t* req_to_lora, int32_t* num_segments, int32_t* tile_info,
                                int32_t* tile_rows, int32_t* num_tiles, int32_t max_tiles,
                                hipStream_t stream);

/*
 * lora_shrink (Ascend walkthrough s2.2-s2.3, first product; SGLang
 * run_lora_a_sgemm): for every sorted position p of segment s with adapter
 * i = req_to_lora[s] and padded rank rp = rank[i]
 *     S[p, sl, j] = sum_k x[sorted_idx[p], k] * A_i[sl*rp + j, k]   (j < rp)
 *     S[p, sl, j] = 0                                                (rp <= j < r_max)
 * x  device [M, ldx] (dtype of w), row m = token m.
 * S  device fp32 [M, n_slices, r_max], rows in sorted order; rows past the
 *    last segment are not written.
 * workspace device, lora_workspace_size(w, M) bytes (zeroed once).
 */
lora_status lora_shrink(const lora_weights_t* w, const void* x, int64_t ldx, int32_t M,
                        const lora_segments_t* seg, float* S, void* workspace,
                        size_t workspace_bytes, hipStream_t stream);

/*
 * lora_expand_add (Ascend walkthrough s2.3, second product added to the base
 * rows; SGLang run_lora_b_sgemm with output offsets): for sorted position p
 * of segment s (adapter i, padded rank rp), slice sl and column n in
 * [slice_offsets[sl], slice_offsets[sl+1]):
 *     y[sorted_idx[p], n] += sum_{j < rp} S[p, sl, j] * B_i[n, j]
 * y  device [M, ldy], updated in place; rows of tokens without an adapter
 *    and of rank-0 slots are neither read nor written.  An output column
 *    offset (a sharded LM head, one slice of a fused output) is expressed by
 *    offsetting the y pointer.
 */
lora_status lora_expand_add(const lora_weights_t* w, const float* S, int32_t M,
                            const lora_segments_t* seg, void* y, int64_t ldy,
                            hipStream_t stream);

/*
 * lora_shrink_expand_add: both products in one call, y += (x A_i^T) B_i^T
 * per token (Ascend walkthrough s2.1 "fused LoRA operator").  For
 * M <= LORA_DECODE_MAX_M it is one kernel launch in which S never leaves
 * the chip except as fp32 partial sums exchanged between workgroups through
 * `workspace`; for larger M it runs lora_shrink then lora_expand_add with S
 * held in `workspace`.
 */
lora_status lora_shrink_expand_add(const lora_weights_t* w, const void* x, int64_t ldx,
                                   int32_t M, const lora_segments_t* seg, void* y, int64_t ldy,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * lora_linear_fused: the base layer and its LoRA delta written together
 * (Ascend walkthrough s1.1, the layer output x W^T + (x A^T) B^T; SGLang
 * "LoRA Layers" page, structure diagram: base output plus LoRA delta):
 *     y[m, n] = sum_k x[m, k] W[n, k] + sum_{j < rp} S[p, sl, j] B_i[n, j]
 * for every token m (sorted position p, adapter i, slice sl holding n); the
 * delta term is absent for tokens without an adapter and for rank-0 slots.
 * Two launches: lora_shrink into `workspace`, then one bf16 MFMA product
 * whose epilogue adds S B_i^T before the single bf16 rounding of y.
 * W  device bf16 [n_total, ldw] row-major (row n = output column n, the
 *    slices of w stacked in order); ldw >= K, ldw % 8 == 0, 16-byte aligned.
 * x  device bf16 [M, ldx]; y device bf16 [M, ldy], overwritten (never read).
 * seg  segment table of the batch (lora_build_segments).
 * workspace  lora_workspace_size(w, M) bytes, as lora_shrink.
 * Only bf16 tables: LORA_UNSUPPORTED for fp32.
 */
lora_status lora_linear_fused(const lora_weights_t* w, const void* W, int64_t ldw,
                              const void* x, int64_t ldx, int32_t M, const lora_segments_t* seg,
                              void* y, int64_t ldy, void* workspace, size_t workspace_bytes,
                              hipStream_t stream);

/*
 * lora_fused_decode: the whole decode path in one kernel launch (Ascend
 * walkthrough s2.1 "fused LoRA operator"; s2.3 grouping by id; s1.2 decode,
 * where every token may carry a different adapter).  For
 * 1 <= M <= LORA_DECODE_MAX_M tokens:
 *     y[m] += (x[m] A_i^T) B_i^T      with i = ids[m], for every token whose
 *                                     id lies in [0, L), whose slot has a
 *                                     non-zero rank and whose adapter is
 *                                     enabled; other rows are untouched.
 * Every workgroup groups the batch by adapter itself (the order
 * lora_build_segments produces), so no segment table has to exist before
 * the call.  When sorted_idx is not NULL the launch also writes the segment
 * table and tile schedule of the batch, bit-identical to what
 * lora_build_segments(ids, adapter_enabled, M, L, ...) writes, so later calls
 * on the same batch (other layers) can use lora_shrink_expand_add with it;
 * the seven table pointers are then all required and max_tiles must be at
 * least lora_tile_capacity(M, L).
 *   ids device [M] int32; adapter_enabled device [L] or NULL;
 *   x device [M, ldx]; y device [M, ldy] updated in place;
 *   workspace as for lora_shrink_expand_add (same size, same rules: zeroed
 *   once, left ready for the next call; calls sharing it are ordered on
 *   one stream).
 * M == 0 writes the empty table (when asked) and nothing else;
 * M > LORA_DECODE_MAX_M returns LORA_UNSUPPORTED (use lora_build_segments
 * and lora_shrink_expand_add).
 */
lora_status lora_fused_decode(const lora_weights_t* w, const int32_t* ids,
                              const int32_t* adapter_enabled, const void* x, int64_t ldx,
                              int32_t M, void* y, int64_t ldy, int32_t* sorted_idx,
                              int32_t* seg_indptr, int32_t* req_to_lora, int32_t* num_segments,
                              int32_t* tile_info, int32_t* tile_rows, int32_t* num_tiles,
                              int32_t max_tiles, void* workspace, size_t workspace_bytes,
                              hipStream_t stream);

/*
 * lora_fused_decode_noalloc: lora_fused_decode for callers that cannot
 * allocate device memory or pass a workspace (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  Same arguments,
 * results and table outputs as lora_fused_decode, without `workspace`: the
 * exchange slots live in a fixed array of LORA_NOALLOC_SCRATCH_BYTES per GPU
 * inside the library, held until the process ends and found on the first
 * call made on each device.  The call allocates and frees nothing.
 *   error_word  device int32, or NULL: error bits (LORA_DEVERR_*) are OR-ed
 *               into it (sticky; the caller clears it); NULL drops them.
 * The array's share of a table is 256 + 8 * 64 * ceil(K / 1024) * n_slices
 * * r_max bytes (M plays no part); a table that needs more than
 * LORA_NOALLOC_SCRATCH_BYTES returns LORA_UNSUPPORTED before any launch.
 * Nothing in the array needs clearing between calls (each launch tags what
 * it writes), but every call on one GPU uses the same array: calls that
 * overlap in time on one GPU (other streams, other threads) race and must
 * not be issued.
 */
#define LORA_NOALLOC_SCRATCH_BYTES (1 << 20)

lora_status lora_fused_decode_noalloc(const lora_weights_t* w, const int32_t* ids,
                                      const int32_t* adapter_enabled, const void* x, int64_t ldx,
                                      int32_t M, void* y, int64_t ldy, int32_t* sorted_idx,
                                      int32_t* seg_indptr, int32_t* req_to_lora,
                                      int32_t* num_segments, int32_t* tile_info,
                                      int32_t* tile_rows, int32_t* num_tiles, int32_t max_tiles,
                                      int32_t* error_word, hipStream_t stream);

/* ---------------------------------------------------------------- embedding LoRA */

/*
 * Embedding LoRA (SGLang "LoRA Layers" page, VocabParallelEmbeddingWithLoRA):
 * the A side is an embedding lookup, A_i (rank, vocab) read by token id; the
 * B side is the usual expand with B_i (emb, rank) into the base embedding
 * rows.  The table is a lora_weights_t with K = vocab, one slice of width
 * emb, planned with lora_table_plan as usual, and filled by
 * lora_pack_embedding_adapter, which stores A transposed so that a lookup
 * reads one contiguous row:
 *   A rows  A + a_off[i] : [vocab, rank_pad] row-major, row t = column t of
 *                          A_i, zero past the true rank;
 *   B rows  B + b_off[i] : [emb, rank_pad] row-major (as lora_pack_adapter).
 *   A_src device [rank, vocab] row-major; B_src device [emb, rank].
 * rank == 0 writes nothing.  vocab must be a multiple of 8 (as every K).
 */
lora_status lora_pack_embedding_adapter(int32_t dtype, int32_t vocab, int64_t emb, int32_t rank,
                                        int32_t rank_pad, const void* A_src, const void* B_src,
                                        void* A_dst, void* B_dst, hipStream_t stream);

/*
 * lora_embedding_shrink: the lookup side (the page's run_lora_a_embedding).
 * For sorted position p of segment s (adapter i, padded rank rp) and token
 * m = sorted_idx[p] with token id t = tokens[m]:
 *     S[p, j] = A_i[j, t]      (j < rp)
 *     S[p, j] = 0              (rp <= j < r_max, and every j when t lies
 *                               outside [0, vocab): the page masks such added
 *                               tokens and has no LoRA for them)
 * tokens device [M] int32; S device fp32 [M, r_max], rows in sorted order;
 * rows past the last segment are not written.  w must have n_slices == 1.
 * lora_expand_add(w, S, M, seg, y, ldy, stream) then adds S B_i^T to the
 * base embedding rows y [M, emb].
 */
lora_status lora_embedding_shrink(const lora_weights_t* w, const int32_t* tokens, int32_t M,
                                  const lora_segments_t* seg, float* S, hipStream_t stream);

/*
 * lora_embedding_decode: the whole embedding-LoRA path for a small batch in
 * one kernel launch (the lookup of lora_embedding_shrink and the expand of
 * lora_expand_add, with the grouping of lora_fused_decode).  For
 * 1 <= M <= LORA_DECODE_MAX_M:
 *     y[m, n] += sum_j A_i[j, t] B_i[n, j]     i = ids[m], t = tokens[m]
 * for tokens with an (enabled, non-empty) adapter and 0 <= t < vocab; other
 * rows are not written.  Every workgroup groups the batch by adapter itself
 * and reads its tokens' S rows straight from the transposed A table, so no
 * workgroup waits for another and no workspace is needed.  When sorted_idx
 * is not NULL the launch also writes the segment table and tile schedule
 * (as lora_fused_decode).  w must be an embedding table (n_slices == 1, A
 * packed by lora_pack_embedding_adapter).  M == 0 writes the empty table
 * (when asked) and nothing else; M > LORA_DECODE_MAX_M returns
 * LORA_UNSUPPORTED (use lora_build_segments, lora_embedding_shrink and
 * lora_expand_add).
 */
lora_status lora_embedding_decode(const lora_weights_t* w, const int32_t* ids,
                                  const int32_t* adapter_enabled, const int32_t* tokens,
                                  int32_t M, void* y, int64_t ldy, int32_t* sorted_idx,
                                  int32_t* seg_indptr, int32_t* req_to_lora,
                                  int32_t* num_segments, int32_t* tile_info, int32_t* tile_rows,
                                  int32_t* num_tiles, int32_t max_tiles, hipStream_t stream);

/* ---------------------------------------------------------------- MoE LoRA */

/*
 * Dense per-expert stacks (SGLang "LoRA + MoE" page, LoRAInfo), padded rank r
 * (multiple of 16, <= 64) shared by every adapter; rows past an adapter's
 * true rank are zero.
 *   A_gu [L, E, r, H]   B_gu [L, E, 2I, r]   A_d [L, E, r, I]   B_d [L, E, H, r]
 * shared_outer != 0 (the page's experts_shared_outer_loras): the outer,
 * hidden-side stacks have one expert slot shared by every expert,
 *   A_gu [L, 1, r, H]   B_d [L, 1, H, r],
 * while B_gu and A_d stay per expert.
 * adapter_enabled device [L]: 0 turns an adapter's deltas off.
 */
typedef struct lora_moe_weights {
    int32_t dtype;   /* lora_dtype */
    int32_t L, E, H, I, r;
    int32_t shared_outer;
    const void* A_gu;
    const void* B_gu;
    const void* A_d;
    const void* B_d;
    const int32_t* adapter_enabled;
} lora_moe_weights_t;

/*
 * Alignment result (SGLang "MoE LoRA Alignment"), device buffers owned by the
 * caller; max_tokens_padded is a multiple of block_size_m and at least
 * lora_moe_align_capacity(M, topk, E, block_size_m).
 */
typedef struct lora_moe_align_buffers {
    int32_t* sorted_token_ids;   /* [L, max_tokens_padded]: flat pairs m*topk+k, sentinel M*topk */
    int32_t* expert_ids;         /* [L, max_tokens_padded / block_size_m]: -1 for unused blocks */
    int32_t* ntpp;               /* [L]: padded list length per adapter */
    int32_t max_tokens_padded;
    int32_t block_size_m;
} lora_moe_align_t;

/* Smallest valid max_tokens_padded: M*topk + E*(block_size_m-1), rounded up to a block. */
int32_t lora_moe_align_capacity(int32_t M, int32_t topk, int32_t E, int32_t block_size_m);

/*
 * lora_moe_align: per adapter l (enabled, with pairs), experts ascending,
 * the pairs f = m*topk + k with ids[m] == l and topk_ids[m, k] == e in
 * increasing f, each (l, e) bucket padded with the sentinel M*topk to a
 * multiple of block_size_m; expert_ids records e per block.  Disabled or
 * idle adapters get ntpp = 0 and a row of sentinels.  Ids outside [0, L)
 * belong to no list.
 *   topk_ids device [M, topk] int32 in [0, E); ids device [M] (-1 = none);
 *   adapter_enabled device [L];
 *   sorted_token_ids device [L, max_tokens_padded] (out);
 *   expert_ids device [L, max_tokens_padded / block_size_m] (out, -1 for
 *       unused blocks);
 *   ntpp device [L] (out): padded list length per adapter.
 * One workgroup per adapter.  M*topk <= 2^24, E <= 256, topk <= 16,
 * block_size_m a multiple of 16 in [16, 256], max_tokens_padded a multiple
 * of block_size_m and at least lora_moe_align_capacity(M, topk, E,
 * block_size_m).  The outputs are the fields of a lora_moe_align_t that the
 * two delta calls read.
 */
lora_status lora_moe_align(const int32_t* topk_ids, const int32_t* ids,
                           const int32_t* adapter_enabled, int32_t M, int32_t topk, int32_t E,
                           int32_t L, int32_t block_size_m, int32_t max_tokens_padded,
                           int32_t* sorted_token_ids, int32_t* expert_ids, int32_t* ntpp,
                           hipStream_t stream);

/*
 * Bytes of device workspace needed by the two MoE delta calls.  As for
 * lora_workspace_size: zero it once (lora_workspace_init) before its first
 * use and order the calls that share it on one stream.  With bf16 weights a
 * delta call is one launch whose expand workgroups wait (bounded) for the
 * shrink workgroups' partials in the workspace; a wait that runs out sets
 * LORA_DEVERR_WAIT in the workspace's error word (lora_read_device_error).
 */
size_t lora_moe_workspace_size(const lora_moe_weights_t* w, int32_t max_tokens_padded);

/*
 * lora_moe_gate_up_add (stage 1.5, before the activation):
 *   cache1[f, :] += B_gu[l, e] (A_gu[l, e] x[f / topk])
 * for every aligned pair f of adapter l in a block of expert e.
 * x device [M, ldx]; cache1 device [M*topk, ld1] with 2I columns.
 */
lora_status lora_moe_gate_up_add(const lora_moe_weights_t* w, const void* x, int64_t ldx,
                                 int32_t M, int32_t topk, const lora_moe_align_t* align,
                                 void* cache1, int64_t ld1, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream);

/*
 * lora_moe_silu_and_mul (stage 2): cache2[f, j] = silu(cache1[f, j]) * cache1[f, I + j],
 * silu(z) = z / (1 + exp(-z)), for f < P, j < I.
 */
lora_status lora_moe_silu_and_mul(int32_t dtype, const void* cache1, int64_t ld1, void* cache2,
                                  int64_t ld2, int32_t P, int32_t I, hipStream_t stream);

/*
 * lora_moe_down_add (stage 3.5, before the reduce):
 *   cache3[f, :] += B_d[l, e] (A_d[l, e] cache2[f])
 * cache2 device [M*topk, ld2] with I columns; cache3 device [M*topk, ld3] with H columns.
 */
lora_status lora_moe_down_add(const lora_moe_weights_t* w, const void* cache2, int64_t ld2,
                              int32_t M, int32_t topk, const lora_moe_align_t* align,
                              void* cache3, int64_t ld3, void* workspace, size_t workspace_bytes,
                              hipStream_t stream);

/*
 * lora_moe_topk_reduce (final reduce): out[m, :] = sum_k w[m, k] cache3[m*topk + k, :],
 * fp32 sum, one rounding.  topk_weights device fp32 [M, topk].
 */
lora_status lora_moe_topk_reduce(int32_t dtype, const void* cache3, int64_t ld3,
                                 const float* topk_weights, void* out, int64_t ldo, int32_t M,
                                 int32_t topk, int32_t H, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MLORA_H */
