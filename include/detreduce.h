/*
 * libdetreduce: deterministic, batch-invariant fp32 reduction of many
 * contributions into shared destinations, for AMD Instinct MI355X (gfx950).
 *
 * It replaces many-writer atomicAdd accumulation.  The pages behind this
 * library name that pattern as the nondeterminism to remove: several writers
 * adding into one address, with the arrival order deciding the last bits
 * (bitwise-determinism interview note, table "where nondeterminism comes
 * from", multiple-writers row; DeepSeek-V4 book ch. 9, "atomicAdd" glossary
 * entry).  Their fix is one private slot per writer, merged in a fixed order.
 *
 * THE DEFINED ORDER (every deterministic entry point follows it)
 *   1. The contributions of one destination are ordered by source id (ties by
 *      input position).  This is a stable sort by (destination, source id),
 *      as in the DeepSeek-V4 MoE backward (ch. 9, section 3.2).
 *   2. T(v_0..v_{L-1}): chunks of 8 consecutive contributions are summed left
 *      to right, starting from the first element.  The chunk sums are combined
 *      by a balanced pairwise tree that splits at the largest power of two
 *      strictly below the chunk count, left part first.
 *   3. Arithmetic is IEEE binary32 with round to nearest even.  There is no
 *      fused multiply-add and no flush of subnormals.  A product (the combine
 *      gate times a row) is rounded to fp32 before it is added.
 *   Because the tree splits only at aligned powers of two, any division of a
 *   destination's contributions into aligned 2^m-chunk tiles gives the same
 *   bits.  So results depend neither on the grid, the workgroup size or the
 *   tile size, nor on which other destinations or tokens are in the batch
 *   (batch invariance: DeepSeek-V4 book ch. 9, glossary, "batch invariant" and
 *   "deterministic").
 *
 * CONVENTIONS
 *   - Every data pointer is a DEVICE pointer owned by the caller.  The library
 *     allocates no memory.  Scratch space comes from caller workspaces sized
 *     by the *_workspace_size functions; the one exception is
 *     dr_combine_fingerprinted_noalloc, whose scratch is a static device array
 *     of the library.
 *   - Every call is asynchronous on the given HIP stream and does not
 *     synchronise, apart from dr_workspace_status and dr_read_status.
 *   - Argument errors are returned synchronously and nothing is launched.
 *     Bad values inside device arrays (an index out of range) are detected by
 *     the kernels.  They set a device status word, and the call then writes
 *     none of its outputs that accumulate (fail closed: the call refuses to run
 *     rather than silently giving a different result; Megatron-LM determinism
 *     reference, section 1.2, "fail closed").  There is never a fallback to an
 *     unordered or atomic path.
 *   - Layouts are row-major and contiguous.  Row data must be 16-byte aligned,
 *     and `hidden` must be a multiple of 8 for bf16 or 4 for fp32.
 *   - bf16 data are raw bfloat16 values.  They are widened to fp32 exactly.
 *   - The library reads no environment variables.  Launch shapes are fixed
 *     functions of the arguments.  dr_set_launch_params (thread-local) lets
 *     tests vary them, which by construction cannot change any output bit.
 *   - The *_atomic entry points are deliberately NONDETERMINISTIC baselines
 *     with the same shapes.  They use hardware fp32 atomic adds, the pattern
 *     being replaced (Megatron-LM determinism reference, section 3.1 op
 *     catalog: the default unpermute path is an atomic scatter_add_).
 */
#ifndef DETREDUCE_H
#define DETREDUCE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dr_status {
    DR_OK = 0,
    DR_ERR_INVALID_ARGUMENT = 1,   /* null/misaligned pointer, bad size or shape */
    DR_ERR_UNSUPPORTED = 2,        /* valid request this library does not implement */
    DR_ERR_WORKSPACE_TOO_SMALL = 3,
    DR_ERR_INDEX_OUT_OF_RANGE = 4, /* device-detected: an index outside its range */
    DR_ERR_HIP = 5,                /* a HIP runtime call failed */
    DR_ERR_BAD_PLAN = 6            /* device-detected: perm/seg_offsets are inconsistent */
} dr_status;

typedef enum dr_dtype { DR_F32 = 0, DR_BF16 = 1 } dr_dtype;

/* KV cache layouts of dr_decode_attention. */
typedef enum dr_kv_layout {
    DR_KV_TOKEN_MAJOR = 0, /* [batch, max_seq_len, num_kv_heads, head_dim] */
    DR_KV_HEAD_MAJOR = 1   /* [batch, num_kv_heads, max_seq_len, head_dim] */
} dr_kv_layout;

/* Launch shape overrides, for tests of launch invariance.  A zero field keeps
 * the library default.  The setting is thread-local. */
typedef struct dr_launch_params {
    int32_t grid_blocks;        /* workgroups of the persistent kernels (index_add reduce and tile
                                   combine, split-K partials, fingerprint), 1 .. 65536 */
    int32_t tile_chunks_log2;   /* index_add tile = 2^m chunks of 8 rows, m in [3, 7] (default 5) */
    int32_t sort_tile_log2;     /* radix sort keys per workgroup = 2^m, m in [8, 13] (default: about
                                   n / 512, clamped to that range) */
    int32_t chunks_in_flight;   /* index_add: chunks of 8 rows loaded at once per lane group, 1 or 2
                                   (default 1) */
    int32_t splitk_stream;      /* split-K partials for thin N: 1 = the streaming kernel where it
                                   applies (the default), 2 = always the general tile kernel */
} dr_launch_params;

/* Human-readable name of a status code.  Never NULL. */
const char* dr_status_string(dr_status s);

/* Detail of the last error returned on this thread ("" if none).  Never NULL. */
const char* dr_last_error(void);

/* Library ABI version (major * 100 + minor). */
int32_t dr_version(void);

/* Sets (p != NULL) or resets (p == NULL) this thread's launch overrides.
 * Returns DR_ERR_INVALID_ARGUMENT for out-of-range fields, leaving the
 * previous setting in place. */
dr_status dr_set_launch_params(const dr_launch_params* p);

/* Measurement hook (thread-local).  With two events set, every later
 * index_add-family call on this thread (dr_index_add, dr_index_add_fingerprinted,
 * dr_sparse_attn_dk) records reduce_begin on its stream just before its ordered
 * reduction kernels (segmented reduce, tile combine) and reduce_end just after,
 * so a caller can time the reduction apart from the sort and the plan.  The
 * events stay owned by the caller.  Both NULL turns the hook off; one NULL is
 * DR_ERR_INVALID_ARGUMENT. */
dr_status dr_set_phase_events(hipEvent_t reduce_begin, hipEvent_t reduce_end);

/* ------------------------------------------------------------------------
 * Stable sort of contributions by destination.
 *
 * Defines the order of contributions: by (dest, src_id), ties by input
 * position.  This is the DeepSeek-V4 MoE backward (ch. 9, section 3.2): tokens
 * are sorted by (expert_id, original_token_id) and merged in sorted order.
 * Stable sorts are naturally deterministic (Megatron-LM determinism
 * reference, section 3, naturally deterministic operations).
 *
 *   dest[n]          destination of each contribution, 0 <= dest < num_dests.
 *   src_id[n]        source id of each contribution, 0 <= src_id < src_id_bound;
 *                    NULL means src_id[i] = i (then src_id_bound is ignored).
 *   perm[n]          OUT: perm[r] = input position of the r-th contribution
 *                    in sorted order.
 *   seg_offsets[num_dests+1]  OUT: CSR offsets; the contributions of d are
 *                    perm[seg_offsets[d] .. seg_offsets[d+1]).
 *   inv_perm[n]      OUT, optional (NULL to skip): inv_perm[perm[r]] = r.  For
 *                    MoE dispatch with dest = expert and i = t*k + j, this is
 *                    the row of (t, j) in the expert-major layout.
 *   ws, ws_bytes     workspace of at least dr_sort_workspace_size(n,
 *                    num_dests, src_id ? src_id_bound : 0) bytes, 16-byte
 *                    aligned.  The first 256 bytes hold the call's device
 *                    status word (see dr_workspace_status).
 * Integer result, exactly reproducible.  n may be 0.  n < 2^31.
 * An out-of-range dest or src_id sets the status word to
 * DR_ERR_INDEX_OUT_OF_RANGE; perm, seg_offsets and inv_perm are then undefined.
 * ---------------------------------------------------------------------- */
size_t dr_sort_workspace_size(int64_t n, int32_t num_dests, int32_t src_id_bound);
dr_status dr_sort_by_dest(const int32_t* dest, const int32_t* src_id, int32_t src_id_bound, int64_t n,
                          int32_t num_dests, int32_t* perm, int32_t* seg_offsets, int32_t* inv_perm,
                          void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * MoE token combine (unpermute): out[t] = T over the token's k contributions.
 *
 * Contribution (t, j) is fl32(gates[t*k+j] * rows[row_of[t*k+j]]), taken in
 * ascending row order (ties by slot j).  With the expert-major layout of the
 * dispatch sort, this is expert-id order, which is the same for every expert-
 * parallel size (bitwise-determinism interview note: every EP size goes
 * through one fp32 reduction tree).  The operation is the MoE token
 * unpermute of the Megatron-LM op catalog (determinism reference, section
 * 3.1) and the merge step of the DeepSeek-V4 MoE backward (ch. 9, section 3.2).
 *
 *   rows[num_rows, hidden]  expert outputs, fp32 or bf16.
 *   row_of[T, k], gates[T, k]  int32 row ids and fp32 gates.  1 <= k <= 64.
 *   out[T, hidden]          OUT, fp32, written (not accumulated).
 *   dev_status              optional device int32 status word (see
 *                           dr_read_status).  If a token references a row
 *                           outside [0, num_rows), that token's output row is
 *                           set to NaN, no row outside the buffer is read, and
 *                           an index error bit is OR-ed into *dev_status.  The
 *                           library never clears the word; the caller zeroes it.
 * ---------------------------------------------------------------------- */
dr_status dr_combine(const void* rows, dr_dtype rows_dtype, int64_t num_rows, int64_t hidden,
                     const int32_t* row_of, const float* gates, int64_t T, int32_t k, float* out,
                     int32_t* dev_status, hipStream_t stream);

/* The same combine, also writing dr_fingerprint(out) to *out_hash: every
 * workgroup hashes the bytes it stores, so the output is not read back.
 * out_hash and the output bits equal those of dr_combine followed by
 * dr_fingerprint.  ws: >= dr_combine_fingerprinted_workspace_size() bytes,
 * 16-byte aligned. */
size_t dr_combine_fingerprinted_workspace_size(dr_dtype rows_dtype, int64_t hidden, int64_t T);
dr_status dr_combine_fingerprinted(const void* rows, dr_dtype rows_dtype, int64_t num_rows, int64_t hidden,
                                   const int32_t* row_of, const float* gates, int64_t T, int32_t k, float* out,
                                   uint64_t* out_hash, void* ws, size_t ws_bytes, int32_t* dev_status,
                                   hipStream_t stream);

/* dr_combine_fingerprinted without a workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, results and bits as
 * dr_combine_fingerprinted, minus ws and ws_bytes; the library allocates
 * nothing and calls no allocating routine.  Its scratch (one fingerprint
 * partial per combine workgroup) is a static 1 MiB device array of the
 * library, of which every GPU the call runs on holds a copy until the process
 * ends.  A call whose scratch would exceed it (T * column slices above about
 * 1,000,000 wavefronts for k <= 8, half that for k > 8: e.g. more than 65,536
 * tokens of 7168 bf16 columns) returns DR_ERR_UNSUPPORTED and launches
 * nothing.  Calls on one GPU share its copy: calls that overlap on one GPU
 * (different streams or host threads) race and must be ordered by the caller;
 * calls in one stream are ordered already. */
dr_status dr_combine_fingerprinted_noalloc(const void* rows, dr_dtype rows_dtype, int64_t num_rows, int64_t hidden,
                                           const int32_t* row_of, const float* gates, int64_t T, int32_t k, float* out,
                                           uint64_t* out_hash, int32_t* dev_status, hipStream_t stream);

/* ------------------------------------------------------------------------
 * index_add: out[d] = out[d] + T(src rows i with index[i] == d, in order of i).
 *
 * This is torch's index_add_(0, index, src), which the Megatron-LM op catalog
 * (determinism reference, section 3.1) uses for the deterministic MoE
 * unpermute and which also forms the vocab-parallel embedding backward.  The
 * DeepSeek-V4 sparse-attention backward (ch. 9, section 3.1) accumulates key
 * gradients of many queries into shared keys in the same way.  The old
 * destination value is added once, last; rows with no contribution are not
 * written (collision-free final write).
 *
 *   out[num_dests, hidden]  fp32, accumulated in place.
 *   src[n, hidden]          fp32 or bf16 contributions.
 *   index[n]                int32 destinations.
 *   perm, seg_offsets       either both NULL (the call sorts internally), or
 *                           both from dr_sort_by_dest(index, src_id = NULL) on
 *                           the same index (a reused plan).  A given plan is
 *                           checked on the device: anything but that stable
 *                           sort (rows in the wrong segment, out of source
 *                           order, repeated or missing) is refused.
 *   ws, ws_bytes            workspace >= dr_index_add_workspace_size(), 16-byte
 *                           aligned; the first 256 bytes are the status word.
 * Device-detected errors (index out of range, inconsistent plan) leave out
 * untouched and are reported by dr_workspace_status.
 * ---------------------------------------------------------------------- */
size_t dr_index_add_workspace_size(int64_t n, int32_t num_dests, int64_t hidden);
dr_status dr_index_add(float* out, int32_t num_dests, int64_t hidden, const void* src, dr_dtype src_dtype,
                       int64_t n, const int32_t* index, const int32_t* perm, const int32_t* seg_offsets,
                       void* ws, size_t ws_bytes, hipStream_t stream);

/* dr_index_add that keeps the destination's fingerprint current.  The
 * fingerprint (dr_fingerprint's definition) is a wrapping sum of position-keyed
 * word terms, so rewriting a row changes it by the new terms minus the old
 * ones.  The reduce kernels form that change from the values they already
 * hold for the read-modify-write, and never read the untouched rows: a step's
 * byte-wise check ("how to verify" in the bitwise-determinism interview note)
 * costs the touched rows only.
 *   inout_hash   device uint64: on entry dr_fingerprint of out as it is; on
 *                return (stream order) dr_fingerprint of the updated out.
 *                When the call fails closed, out and *inout_hash both stay
 *                as they were.
 * Other arguments as dr_index_add. */
dr_status dr_index_add_fingerprinted(float* out, int32_t num_dests, int64_t hidden, const void* src,
                                     dr_dtype src_dtype, int64_t n, const int32_t* index, const int32_t* perm,
                                     const int32_t* seg_offsets, uint64_t* inout_hash, void* ws, size_t ws_bytes,
                                     hipStream_t stream);

/* ------------------------------------------------------------------------
 * Sparse-attention key gradient with the contributions formed on the fly:
 *   dK[key] = dK[key] + T(fl32(dS[q][j] * Q[q]) over the (q, j) with
 *             key_idx[q][j] == key, in order of q * topk + j).
 *
 * The backward of DeepSeek-V4's sparse attention (ch. 9, section 3.1): every
 * query selected topk keys, and a selected key's gradient sums, over the
 * queries that chose it, the query row scaled by its score gradient.  This is
 * dr_index_add over the contributions c[q*topk + j] = fl32(dS[q][j] * Q[q])
 * (each element rounded once, never fused into the add), computed inside the
 * reduction, so the [num_queries * topk, head_dim] contribution matrix is
 * never written or read.  Any softmax scale is folded into dS by the caller.
 *
 *   dK[num_keys, head_dim]    fp32, accumulated in place; keys no query
 *                             selected are not written.
 *   Q[num_queries, head_dim]  fp32 or bf16 rows (16-byte aligned; head_dim a
 *                             multiple of 4 / 8).
 *   dS[num_queries, topk]     fp32 score gradients.
 *   key_idx[num_queries, topk] int32 selected keys.
 *   perm, seg_offsets         both NULL (the call sorts key_idx), or both from
 *                             dr_sort_by_dest(key_idx, src_id = NULL) on the
 *                             same key_idx (a plan reused across calls).
 *   ws, ws_bytes              >= dr_sparse_attn_dk_workspace_size(), 16-byte
 *                             aligned; the first 256 bytes are the status word.
 * num_queries * topk must be below 2^31.  A key index out of range (or an
 * inconsistent plan) leaves dK untouched and is reported by
 * dr_workspace_status.
 * ---------------------------------------------------------------------- */
size_t dr_sparse_attn_dk_workspace_size(int64_t num_queries, int32_t topk, int32_t num_keys, int64_t head_dim);
dr_status dr_sparse_attn_dk(float* dK, int32_t num_keys, int64_t head_dim, const void* Q, dr_dtype q_dtype,
                            const float* dS, const int32_t* key_idx, int64_t num_queries, int32_t topk,
                            const int32_t* perm, const int32_t* seg_offsets, void* ws, size_t ws_bytes,
                            hipStream_t stream);

/* ------------------------------------------------------------------------
 * Split-K contraction into private per-split buffers.
 *
 * partials[s] = X_s^T * dY_s for split s = tokens [s*c, min(K, (s+1)*c)),
 * c = ceil(K / splits).  Each split writes its own buffer and nothing is
 * reduced here (DeepSeek-V4 book ch. 9, section 3.3, mHC backward: every
 * K-split outputs to its own buffer).  Split boundaries are a function of
 * (K, splits) only, never of occupancy (ch. 9, glossary "split-K": a split
 * chosen per batch breaks batch invariance).  Products of bf16 values are
 * summed by bf16 MFMA into fp32, in a fixed order within each split, so a
 * partial is bitwise repeatable and independent of the M/N tiling.
 *
 *   X[K, M], dY[K, N]   bf16.  1 <= splits, and every split non-empty:
 *                       (splits - 1) * c < K.
 *   partials[splits, M, N]  OUT fp32, written.
 * ---------------------------------------------------------------------- */
dr_status dr_splitk_gemm_tn(const void* X, const void* dY, int64_t K, int64_t M, int64_t N, int32_t splits,
                            float* partials, hipStream_t stream);

/* out[e] = T(partials[0][e], ..., partials[splits-1][e]): the deterministic
 * reduce over split ids (DeepSeek-V4 book ch. 9, section 3.3: a dedicated
 * reduce kernel sums the per-split buffers in split-id order).
 *   partials[splits, count] fp32;  out[count] fp32, written. */
dr_status dr_splitk_reduce(const float* partials, int32_t splits, int64_t count, float* out,
                           hipStream_t stream);

/* The same reduce, also writing dr_fingerprint(out) to *out_hash (device
 * uint64).  When count is a multiple of 4, the reduce hashes each 16-byte
 * piece as it stores it, so out is not read back; otherwise out is hashed
 * after the reduce.  out and *out_hash equal those of dr_splitk_reduce
 * followed by dr_fingerprint(out, 4 * count).
 *   ws   >= dr_splitk_reduce_fingerprinted_workspace_size() bytes, 16-byte
 *        aligned, contents on entry do not matter.
 * Errors: the argument checks of dr_splitk_reduce, a null or misaligned
 * out_hash or ws, and a short workspace return an error before any launch. */
size_t dr_splitk_reduce_fingerprinted_workspace_size(int32_t splits, int64_t count);
dr_status dr_splitk_reduce_fingerprinted(const float* partials, int32_t splits, int64_t count, float* out,
                                         uint64_t* out_hash, void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Grouped split with private slots: per group g (an expert),
 *   dW[g] = T over its slots s of  X_s^T dY_s   (slot order),
 * where group g owns tokens [group_offsets[g], group_offsets[g+1]) of the
 * expert-major X and dY and is cut into consecutive slots of split_tokens
 * tokens from its first token (the last slot short).
 *
 * The Megatron Core determinism blog's grouped-GEMM weight-gradient fix, as
 * the bitwise-determinism interview note retells it: several tiles used to
 * accumulate into one address in the epilogue, in arrival order; instead each
 * writer gets a private slot and the slots are merged in a fixed order.  The
 * slot boundaries depend only on the group sizes and split_tokens, never on
 * the grid, so every partial and every dW[g] is repeatable; a group with no
 * tokens gets the zero gradient.
 *
 *   X[K, M], dY[K, N]    bf16 (bit patterns), expert-major token rows.
 *   group_offsets[G+1]   int32, device: non-decreasing within [0, K].
 *   partials             fp32 [partial_slots, M, N], partial_slots >=
 *                        dr_grouped_splitk_max_slots(K, G, split_tokens);
 *                        slot s (in group order) is written for s below the
 *                        slot count, the rest is not touched.
 *   slot_offsets[G+1]    int32, device, written: group g's slots are
 *                        slot_offsets[g] .. slot_offsets[g+1]-1.
 *   ws                   >= dr_grouped_splitk_workspace_size(), 16-byte
 *                        aligned: the status block and the slot table.
 * Offsets that are not non-decreasing within [0, K] set the status word
 * (dr_workspace_status reports DR_ERR_BAD_PLAN) and nothing is computed;
 * dr_grouped_splitk_reduce with the same ws then leaves out untouched.
 * ---------------------------------------------------------------------- */
int64_t dr_grouped_splitk_max_slots(int64_t K, int32_t num_groups, int32_t split_tokens);
size_t dr_grouped_splitk_workspace_size(int64_t K, int32_t num_groups, int32_t split_tokens);
dr_status dr_grouped_splitk_gemm_tn(const void* X, const void* dY, int64_t K, int64_t M, int64_t N,
                                    const int32_t* group_offsets, int32_t num_groups, int32_t split_tokens,
                                    float* partials, int64_t partial_slots, int32_t* slot_offsets, void* ws,
                                    size_t ws_bytes, hipStream_t stream);
/* out[g][e] = T(partials[slot_offsets[g]][e], ..., partials[slot_offsets[g+1]-1][e]), zero for a group
 * with no slot.  out[num_groups, count] fp32, written; ws is the one the partials were made with. */
dr_status dr_grouped_splitk_reduce(const float* partials, int64_t partial_slots, const int32_t* slot_offsets,
                                   int32_t num_groups, int64_t count, float* out, const void* ws,
                                   hipStream_t stream);

/* ------------------------------------------------------------------------
 * The same grouped weight gradient for expert shapes (large M and N), with
 * the slot partials kept in registers: per group g,
 *   dW[g] = T over its slots s of  X_s^T dY_s   (slot order),
 * slots as in dr_grouped_splitk_gemm_tn (consecutive runs of split_tokens
 * tokens from the group's first token).  Same bits as
 * dr_grouped_splitk_gemm_tn followed by dr_grouped_splitk_reduce: each slot's
 * partial is accumulated in token order by the same bf16 MFMA steps, and the
 * slots are summed by the same tree (chunks of 8 slots left to right, then the
 * pairwise tree over the chunk sums).  The partials never reach memory: a
 * workgroup owns a 256 x 128 tile of dW[g] and adds each slot's partial into
 * the chunk's running sum as the slot ends; a group of more than 8 slots
 * leaves its chunk sums in ws, and a merge applies the pairwise tree over them
 * (the private-slot grouped-GEMM weight gradient of the bitwise-determinism
 * interview note, multiple-writers row; Megatron-LM determinism reference,
 * section 3.3, grouped-GEMM weight gradient as a determinism hotspot).
 *
 *   X[K, M], dY[K, N]    bf16 (bit patterns), expert-major token rows, 16-byte
 *                        aligned; M and N multiples of 8 and at most 2^23
 *                        (other shapes: dr_grouped_splitk_gemm_tn).
 *   group_offsets[G+1]   int32, device: non-decreasing within [0, K].
 *   out[G, M, N]         fp32, written; a group with no token gets zeros.
 *   ws                   >= dr_grouped_wgrad_workspace_size(K, G, split_tokens,
 *                        M, N) bytes, 16-byte aligned: the status block, the
 *                        work plan and room for the chunk sums of groups of
 *                        more than 8 slots (at most K / (4 split_tokens) + 1
 *                        tiles of M x N).  Its contents on entry do not matter.
 * Offsets that are not non-decreasing within [0, K] set the status word
 * (dr_workspace_status reports DR_ERR_BAD_PLAN) and out is not written.
 * ---------------------------------------------------------------------- */
size_t dr_grouped_wgrad_workspace_size(int64_t K, int32_t num_groups, int32_t split_tokens, int64_t M, int64_t N);
dr_status dr_grouped_wgrad(const void* X, const void* dY, int64_t K, int64_t M, int64_t N,
                           const int32_t* group_offsets, int32_t num_groups, int32_t split_tokens, float* out,
                           void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Dispatch-side stable permute: out[r] = rows[perm[r] / k] (bytes copied).
 *
 * perm is dr_sort_by_dest's permutation of the T*k (token, slot) assignments
 * by expert, so out holds each expert's tokens contiguously in token order,
 * the layout of the DeepSeek-V4 MoE backward (ch. 9, section 3.2: tokens
 * sorted by (expert_id, original_token_id)).  No arithmetic: exact.
 *   rows[num_rows, row_bytes], out[n, row_bytes]: 16-byte aligned, row_bytes
 *   a multiple of 16.
 *   inv_perm  optional (NULL: the work runs in output order): the sort's
 *             inverse permutation.  Then the copies run in token order and a
 *             token row is read from HBM about once instead of k times; each
 *             output row is still the one perm assigns, written once.
 * A perm entry outside [0, num_rows * k), or an inv_perm entry that perm does
 * not invert, sets *dev_status (when given) and that output row is not written.
 * ---------------------------------------------------------------------- */
dr_status dr_permute_rows(const void* rows, int64_t row_bytes, int64_t num_rows, const int32_t* perm,
                          const int32_t* inv_perm, int64_t n, int32_t k, void* out, int32_t* dev_status,
                          hipStream_t stream);

/* ------------------------------------------------------------------------
 * Batch-invariant decode attention (DeepSeek-V4 book ch. 9, section 2.1).
 *
 * One query token per sequence attends to the sequence's first seq_lens[b]
 * cached keys and values:
 *   out[b, h] = sum_j softmax_j(scale * q[b, h] . k[b, j, h / G]) v[b, j, h / G]
 * with G = num_q_heads / num_kv_heads query heads per KV head (grouped-query
 * attention); a sequence of length 0 gives zeros.  That chapter gives up split-KV
 * decoding because its partition of the keys, and with it the order in which
 * the partial softmax sums merge, follows the batch size and the occupancy.
 * Here the keys of a sequence are cut into chunks of kv_chunk tokens from its
 * first token, whatever the batch: each chunk computes private partials (its
 * maximum, weight sum and weighted value sum per query head) in an order fixed
 * by the chunk alone, and the partials merge in chunk order.  A sequence's
 * output bits therefore depend only on its own q, cache rows, length, scale and
 * kv_chunk: not on the other sequences, the batch size, its position in the
 * batch or the device's size.  kv_chunk >= the sequence length runs the whole
 * sequence serially in one workgroup, the chapter's single-processor prefix.
 * Scores are exact bf16 products summed in fp32 (matrix cores); weights are
 * 2^(t - max) with t = score * scale * log2(e) in fp32.
 *
 *   out          OUT fp32 [batch, num_q_heads, head_dim], 16-byte aligned.
 *   q            bf16 [batch, num_q_heads, head_dim].
 *   k_cache, v_cache  bf16, laid out as kv_layout says: token-major
 *                [batch, max_seq_len, num_kv_heads, head_dim] or head-major
 *                [batch, num_kv_heads, max_seq_len, head_dim].  Rows at or past
 *                a sequence's length are never read.  Both layouts give the
 *                same bits.
 *   seq_lens     int32 [batch], 0 <= seq_lens[b] <= max_seq_len.  A length
 *                outside that range ORs an index error bit into *dev_status
 *                (when given) and that sequence's output rows are not written.
 *   head_dim     128.  num_q_heads / num_kv_heads must be 1, 2, 4, 8 or 16.
 *   max_seq_len  1 .. 2^30.  kv_chunk: a multiple of 64 in [64, 2^20].
 *   ws           >= dr_decode_attention_workspace_size(...) bytes, 16-byte
 *                aligned: one partial slot per (sequence, query head, chunk)
 *                after 256 reserved bytes.  Its contents on entry do not
 *                matter; device errors go to dev_status only (the workspace
 *                holds no status word, so dr_workspace_status does not apply).
 * All pointers must be 16-byte aligned (seq_lens and dev_status 4-byte).
 * ---------------------------------------------------------------------- */
size_t dr_decode_attention_workspace_size(int64_t batch, int32_t num_q_heads, int32_t max_seq_len, int32_t kv_chunk,
                                          int64_t head_dim);
dr_status dr_decode_attention(float* out, const void* q, const void* k_cache, const void* v_cache,
                              dr_kv_layout kv_layout, const int32_t* seq_lens, int64_t batch, int32_t num_q_heads,
                              int32_t num_kv_heads, int64_t head_dim, int32_t max_seq_len, float scale,
                              int32_t kv_chunk, void* ws, size_t ws_bytes, int32_t* dev_status, hipStream_t stream);

/* The kv_chunk an occupancy-driven split-KV heuristic would pick for this batch
 * on the current device: enough chunks to give every compute unit two
 * workgroups, so it CHANGES WITH THE BATCH SIZE.  A deliberately batch-variant
 * baseline, the pattern that chapter rejects; passing it to dr_decode_attention
 * shows the output bits moving with the batch.  Returns 0 on bad arguments. */
int32_t dr_decode_attention_occupancy_chunk(int64_t batch, int32_t num_kv_heads, int32_t max_seq_len);

/* ------------------------------------------------------------------------
 * Byte fingerprint of a tensor, for comparing runs byte for byte rather than
 * by printed values (bitwise-determinism interview note, "how to verify":
 * per-step tensor fingerprints compared byte-wise).  The definition is this
 * library's own:
 *   h = mix(nbytes) + sum_i mix(w_i XOR s_i)   (mod 2^64)
 * w_i is the i-th little-endian 64-bit word of the bytes in logical order,
 * the last word zero-padded; s_i = (i + 1) * 0x9e3779b97f4a7c15 (the states of
 * a SplitMix64 generator started at 0); mix is SplitMix64's finaliser.  +0.0
 * and -0.0, and NaNs with different payloads, hash differently.
 *   data       device pointer, 8-byte aligned (or nbytes == 0).
 *   out_hash   OUT device uint64.
 *   ws         >= dr_fingerprint_workspace_size(nbytes) bytes, 16-byte aligned.
 * ---------------------------------------------------------------------- */
size_t dr_fingerprint_workspace_size(int64_t nbytes);
dr_status dr_fingerprint(const void* data, int64_t nbytes, uint64_t* out_hash, void* ws, size_t ws_bytes,
                         hipStream_t stream);

/* ------------------------------------------------------------------------
 * Status words (these two calls synchronise the stream).
 * A device status word is an int32 of error bits: 1 = an index out of range,
 * 2 = an inconsistent caller-supplied plan.  These calls return DR_OK for 0,
 * DR_ERR_BAD_PLAN if bit 2 is set, else DR_ERR_INDEX_OUT_OF_RANGE.
 * dr_workspace_status reads the word at the head of a sort or index_add
 * workspace, which every call on that workspace clears first.
 * dr_read_status reads a caller-owned word such as dr_combine's.
 * ---------------------------------------------------------------------- */
dr_status dr_workspace_status(const void* ws, hipStream_t stream);
dr_status dr_read_status(const int32_t* dev_status, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Deliberately nondeterministic atomicAdd baselines (same shapes).  The
 * caller initialises out (zero for combine and split-K).  Out-of-range
 * indices are skipped and OR an index error bit into *dev_status when it is
 * not NULL.
 * ---------------------------------------------------------------------- */
dr_status dr_combine_atomic(const void* rows, dr_dtype rows_dtype, int64_t num_rows, int64_t hidden,
                            const int32_t* row_of, const float* gates, int64_t T, int32_t k, float* out,
                            int32_t* dev_status, hipStream_t stream);
dr_status dr_index_add_atomic(float* out, int32_t num_dests, int64_t hidden, const void* src,
                              dr_dtype src_dtype, int64_t n, const int32_t* index, int32_t* dev_status,
                              hipStream_t stream);
dr_status dr_splitk_gemm_tn_atomic(const void* X, const void* dY, int64_t K, int64_t M, int64_t N,
                                   int32_t splits, float* out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DETREDUCE_H */
