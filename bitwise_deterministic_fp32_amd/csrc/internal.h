// Internal declarations shared by the HIP kernels and the C-ABI layer of
// libdetreduce.  Not installed; the public interface is include/detreduce.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "detreduce.h"

namespace dr {

// ---------------------------------------------------------------------------
// Status word bits (int32 at the head of a sort / index_add workspace, or a
// caller-owned word for combine and the atomic baselines).  dr_read_status
// maps them to dr_status codes.
// ---------------------------------------------------------------------------
constexpr int32_t kStatusIndex = 1;  // an index outside its range
constexpr int32_t kStatusPlan = 2;   // a caller-supplied plan is inconsistent
constexpr size_t kStatusBytes = 256;  // status block at the head of a workspace
// Words of the status block: [0] status, [1] total tiles, [2] multi-tile segments.
constexpr int kWordStatus = 0;
constexpr int kWordTiles = 1;
constexpr int kWordMultis = 2;
constexpr int kWordSlots = 1;  // grouped split: private slots in use (its own workspace)

constexpr int kDefaultTileChunksLog2 = 5;
constexpr int kMinTileChunksLog2 = 3;
constexpr int kMaxTileChunksLog2 = 7;
constexpr int kMinSortTileLog2 = 8;
constexpr int kMaxSortTileLog2 = 13;
constexpr int kMaxDigitBits = 9;  // radix digits of up to 9 bits (512 bins)
// Default keys per sort workgroup: about n / 512, clamped to [2^8, 2^13], so
// that small sorts still spread over the whole GPU.  A function of n only.
inline int default_sort_tile_log2(int64_t n) {
    int t = 0;
    while (t < 62 && ((int64_t)1 << t) < n) ++t;
    t -= 9;
    return t < kMinSortTileLog2 ? kMinSortTileLog2 : (t > kMaxSortTileLog2 ? kMaxSortTileLog2 : t);
}

// ---------------------------------------------------------------------------
// Launch configuration in force for the calling thread.
// ---------------------------------------------------------------------------
struct Launch {
    int grid_blocks;       // 0 = default
    int tile_chunks_log2;  // resolved value
    int sort_tile_log2;    // 0 = default_sort_tile_log2(n)
    int chunks_in_flight;  // resolved value (1 or 2)
    bool splitk_stream;    // thin-N split-K partials may use the streaming kernel
    int sort_tile(int64_t n) const { return sort_tile_log2 ? sort_tile_log2 : default_sort_tile_log2(n); }
};
Launch launch_config();

// Error reporting of the C ABI (the thread-local text dr_last_error returns).
dr_status report(dr_status s, const char* fmt, ...);
dr_status report_ok();
dr_status report_hip(hipError_t e, const char* what);
// Argument checks shared by the combine entry points (nothing is launched on
// an error; the error text is set).
dr_status validate_combine(const char* what, const void* rows, dr_dtype rows_dtype, int64_t num_rows, int64_t hidden,
                           const int32_t* row_of, const float* gates, int64_t T, int32_t k, const float* out,
                           const int32_t* dev_status);
int device_cu_count();  // compute units of the current device (cached)

// ---------------------------------------------------------------------------
// Plan records written by the index_add planner
// ---------------------------------------------------------------------------
struct alignas(16) TileRec {
    int32_t dest;     // destination row
    int32_t r_begin;  // sorted positions [r_begin, r_end) of the tile's rows
    int32_t r_end;
    int32_t pslot;    // partial slot, or -1 when the tile is the whole segment
};
struct alignas(16) MultiRec {
    int32_t dest;
    int32_t pslot0;  // first partial slot of the segment's tiles
    int32_t ntiles;
    int32_t pad;
};

// ---------------------------------------------------------------------------
// Host launchers (each defined next to its kernels).  All return hipSuccess or
// the launch error; shapes are validated by the caller.
// ---------------------------------------------------------------------------
hipError_t launch_fill_status(int32_t* status_block, hipStream_t s);

// radix sort pieces
struct SortPass {
    const int32_t* digit_src;  // array the digit is read from (current order)
    int shift;
    int bits;
    const int32_t* dest_in;
    int32_t* dest_out;         // may be null on the last pass if keys are not needed
    const int32_t* src_in;     // null when no explicit source ids remain to carry
    int32_t* src_out;
    const int32_t* val_in;     // null = identity (first pass)
    int32_t* val_out;
    int32_t* inv_out;          // last pass only (optional)
    int32_t* seg_out;          // set when this pass's digit is the whole destination (a single dest
                               // pass): workgroup 0 then writes seg_offsets[0 .. num_dests]
    int32_t num_dests;
    const float* pay_in;       // optional payload moved with the keys (input order on the first pass)
    float* pay_out;            // set together with pay_in; no source ids are carried then
};
hipError_t launch_radix_validate_hist(const int32_t* dest, int32_t num_dests, const int32_t* src_id,
                                      int32_t src_bound, const SortPass& p, int64_t n, int tile_log2,
                                      int32_t* hist, int32_t* tile_flags, hipStream_t s);
hipError_t launch_radix_hist(const SortPass& p, int64_t n, int tile_log2, int32_t* hist, const int32_t* status,
                             hipStream_t s);
// tile_flags non-null (the first pass): one more workgroup folds the tiles'
// index-error flags into the status word, which it thereby sets or clears.
hipError_t launch_radix_scan(int32_t* hist, int64_t nblocks, int bins, int32_t* totals, int32_t* status,
                             const int32_t* tile_flags, hipStream_t s);
hipError_t launch_radix_scatter(const SortPass& p, int64_t n, int tile_log2, const int32_t* hist,
                                const int32_t* totals, const int32_t* status, hipStream_t s);
hipError_t launch_seg_offsets(const int32_t* sorted_dest, int64_t n, int32_t num_dests, int32_t* seg_offsets,
                              const int32_t* status, hipStream_t s);

// index_add planner and reducer
int64_t plan_blocks(int32_t num_dests);
hipError_t launch_plan_count(const int32_t* seg_offsets, int32_t num_dests, int64_t n, int tile_chunks_log2,
                             int32_t* block_sums, int32_t* status, hipStream_t s);
// plan_count for the library's own sort: segment offsets searched in the sorted destinations, written, and counted
hipError_t launch_plan_count_search(const int32_t* sorted_dest, int64_t n, int32_t num_dests, int tile_chunks_log2,
                                    int32_t* seg_offsets, int32_t* block_sums, int32_t* status, hipStream_t s);
hipError_t launch_plan_write(const int32_t* seg_offsets, int32_t num_dests, int tile_chunks_log2,
                             const int32_t* block_sums, TileRec* tiles, MultiRec* multis, int32_t* status,
                             hipStream_t s);
hipError_t launch_plan_validate(const int32_t* perm, const int32_t* seg, const int32_t* index, int64_t n,
                                int32_t num_dests, int32_t* status, hipStream_t s);
// scale != null: source row p contributes fl32(scale[p] * src[p / rows_per_src])
// scale_sorted: scale is in sorted order (scale[r] belongs to sorted position
// r) instead of indexed by source row.
hipError_t launch_segreduce(float* out, int64_t hidden, const void* src, dr_dtype src_dtype, int64_t n,
                            const int32_t* perm, const TileRec* tiles, float* partials, int tile_chunks_log2,
                            int chunks_in_flight, const float* scale, bool scale_sorted, int32_t rows_per_src,
                            int32_t* status, uint64_t* fp_part, hipStream_t s);
hipError_t launch_tilecombine(float* out, int64_t hidden, const float* partials, const MultiRec* multis, int64_t n,
                              int tile_chunks_log2, int32_t* status, uint64_t* fp_part, hipStream_t s);
// Workgroups of the persistent reduce kernels (segreduce, tilecombine); with
// fp_part each of them writes one fingerprint change there.
unsigned persistent_grid();
// hash += sum of nparts fingerprint changes, unless the status word is set.
hipError_t launch_fingerprint_update(const uint64_t* parts, int64_t nparts, const int32_t* status, uint64_t* hash,
                                     hipStream_t s);

// combine
// fp_partials != nullptr: also hash the written output (one partial per workgroup)
hipError_t launch_combine(const void* rows, dr_dtype dt, int64_t num_rows, int64_t hidden, const int32_t* row_of,
                          const float* gates, int64_t T, int32_t k, float* out, int32_t* dev_status, bool atomic,
                          uint64_t* fp_partials, hipStream_t s);
// index_add atomic baseline
hipError_t launch_index_add_atomic(float* out, int32_t num_dests, int64_t hidden, const void* src,
                                   dr_dtype dt, int64_t n, const int32_t* index, int32_t* dev_status,
                                   hipStream_t s);
// split-K
hipError_t launch_splitk_gemm(const uint16_t* X, const uint16_t* dY, int64_t K, int64_t M, int64_t N,
                              int32_t splits, float* out, bool atomic, hipStream_t s);
// fp_part != nullptr (count a multiple of 4): the launch also writes the
// fingerprint terms of out, one partial sum per workgroup
int64_t splitk_reduce_blocks(int32_t splits, int64_t count);
hipError_t launch_splitk_reduce(const float* partials, int32_t splits, int64_t count, float* out, uint64_t* fp_part,
                                hipStream_t s);
// grouped split with private slots: the slot table, then the partials of every slot
hipError_t launch_grouped_splitk_gemm(const uint16_t* X, const uint16_t* dY, int64_t K, int64_t M, int64_t N,
                                      const int32_t* group_offsets, int32_t num_groups, int32_t split_tokens,
                                      int64_t max_slots, int32_t* slot_offsets, int2* ranges, int32_t* status,
                                      float* out, hipStream_t s);
hipError_t launch_grouped_reduce(const float* partials, const int32_t* slot_offsets, int64_t max_slots,
                                 int32_t num_groups, int64_t count, float* out, const int32_t* status,
                                 hipStream_t s);
// grouped-GEMM weight gradient with private slots, slot partials kept in registers (large M and N):
// the plan, the tile kernel and the merge of chunk sums of groups of more than 8 slots
int64_t wgrad_max_chunk_rows(int64_t K, int32_t split);
int64_t wgrad_max_items(int64_t K, int32_t num_groups, int32_t split, int64_t M, int64_t N);
hipError_t launch_wgrad(const uint16_t* X, const uint16_t* dY, int64_t K, int64_t M, int64_t N,
                        const int32_t* group_offsets, int32_t num_groups, int32_t split, float* out,
                        int32_t* status, int32_t* cum_items, int32_t* chunk_base, float* chunks, hipStream_t s);
// dispatch-side permute: out[r] = rows[perm[r] / k]; with inv_perm the work runs in token order
hipError_t launch_permute_rows(const void* rows, int64_t row_bytes, int64_t num_rows, const int32_t* perm,
                               const int32_t* inv_perm, int64_t n, int32_t k, void* out, int32_t* dev_status,
                               hipStream_t s);
// fingerprint
// most workgroups (and partials) of a fingerprint launch: 8 per SIMD of a
// 256-CU device, enough wavefronts to hide the loads behind the hashing
constexpr int kMaxFingerprintBlocks = 8192;
int64_t fingerprint_blocks(int64_t nbytes);
hipError_t launch_fingerprint(const void* data, int64_t nbytes, uint64_t* out, uint64_t* block_partials,
                              hipStream_t s);
// out = mix(nbytes) + sum of nblocks per-workgroup partial sums; group_sums
// holds fingerprint_group_count(nblocks) values for a two-level sum
int64_t fingerprint_group_count(int64_t nblocks);
hipError_t launch_fingerprint_final(const uint64_t* block_partials, int64_t nblocks, int64_t nbytes, uint64_t* out,
                                    uint64_t* group_sums, hipStream_t s);
// number of workgroups (and fingerprint partials) of a fingerprinting combine launch
// (k = 64 gives the largest count, for any k)
// Decode attention: chunk partial slots per sequence, and the two kernels
// (chunk partials, then the ordered merge).  ml holds (max, weight sum) per
// slot, po the weighted value sums (head_dim 128).
int64_t decode_num_chunks(int32_t max_seq_len, int32_t kv_chunk);
hipError_t launch_decode_attention(float* out, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                   const int32_t* seq_lens, int64_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                   int32_t max_seq_len, bool head_major, float scale, int32_t kv_chunk, float2* ml,
                                   float* po, int32_t* status, hipStream_t s);
int64_t combine_fp_blocks(dr_dtype dt, int64_t hidden, int64_t T, int32_t k);

}  // namespace dr

#ifdef __HIPCC__
#include "device.h"
#endif
