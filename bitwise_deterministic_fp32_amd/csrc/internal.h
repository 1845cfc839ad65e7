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

constexpr int kDefaultTileChunksLog2 = 5;
constexpr int kMinTileChunksLog2 = 3;
constexpr int kMaxTileChunksLog2 = 7;
constexpr int kMinSortTileLog2 = 8;
constexpr int kMaxSortTileLog2 = 12;
constexpr int kMaxDigitBits = 9;  // radix digits of up to 9 bits (512 bins)
// Default keys per sort workgroup: about n / 512, clamped to [2^8, 2^12], so
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
    int sort_tile(int64_t n) const { return sort_tile_log2 ? sort_tile_log2 : default_sort_tile_log2(n); }
};
Launch launch_config();
int device_cu_count();  // compute units of the current device (cached)

// ---------------------------------------------------------------------------
// Plan records written by the index_add planner
// ---------------------------------------------------------------------------
struct alignas(16) TileRec {
    int32_t dest;    // destination row
    int32_t chunk0;  // first chunk (of 8 rows) of the tile, relative to the segment start
    int32_t pslot;   // partial slot, or -1 when the tile is the whole segment
    int32_t pad;
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
};
hipError_t launch_radix_validate_hist(const int32_t* dest, int32_t num_dests, const int32_t* src_id,
                                      int32_t src_bound, const SortPass& p, int64_t n, int tile_log2,
                                      int32_t* hist, int32_t* status, hipStream_t s);
hipError_t launch_radix_hist(const SortPass& p, int64_t n, int tile_log2, int32_t* hist, const int32_t* status,
                             hipStream_t s);
hipError_t launch_radix_scan(int32_t* hist, int64_t nblocks, int bins, int32_t* totals, const int32_t* status,
                             hipStream_t s);
hipError_t launch_radix_scatter(const SortPass& p, int64_t n, int tile_log2, const int32_t* hist,
                                const int32_t* totals, const int32_t* status, hipStream_t s);
hipError_t launch_seg_offsets(const int32_t* sorted_dest, int64_t n, int32_t num_dests, int32_t* seg_offsets,
                              const int32_t* status, hipStream_t s);

// index_add planner and reducer
int64_t plan_blocks(int32_t num_dests);
hipError_t launch_plan_count(const int32_t* seg_offsets, int32_t num_dests, int64_t n, int tile_chunks_log2,
                             int32_t* block_sums, int32_t* status, hipStream_t s);
hipError_t launch_plan_write(const int32_t* seg_offsets, int32_t num_dests, int tile_chunks_log2,
                             const int32_t* block_sums, TileRec* tiles, MultiRec* multis, int32_t* status,
                             hipStream_t s);
hipError_t launch_plan_validate(const int32_t* perm, const int32_t* seg, const int32_t* index, int64_t n,
                                int32_t num_dests, int32_t* status, hipStream_t s);
hipError_t launch_segreduce(float* out, int64_t hidden, const void* src, dr_dtype src_dtype, int64_t n,
                            const int32_t* perm, const int32_t* seg_offsets, const TileRec* tiles,
                            float* partials, int tile_chunks_log2, int chunks_in_flight, int32_t* status,
                            hipStream_t s);
hipError_t launch_tilecombine(float* out, int64_t hidden, const float* partials, const MultiRec* multis, int64_t n,
                              int tile_chunks_log2, int32_t* status, hipStream_t s);

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
hipError_t launch_splitk_reduce(const float* partials, int32_t splits, int64_t count, float* out,
                                hipStream_t s);
// fingerprint
int64_t fingerprint_blocks(int64_t nbytes);
hipError_t launch_fingerprint(const void* data, int64_t nbytes, uint64_t* out, uint64_t* block_partials,
                              hipStream_t s);
// out = mix(nbytes) + sum of nblocks per-workgroup partial sums; group_sums
// holds fingerprint_group_count(nblocks) values for a two-level sum
int64_t fingerprint_group_count(int64_t nblocks);
hipError_t launch_fingerprint_final(const uint64_t* block_partials, int64_t nblocks, int64_t nbytes, uint64_t* out,
                                    uint64_t* group_sums, hipStream_t s);
// number of workgroups (and fingerprint partials) of a combine launch
int64_t combine_blocks(dr_dtype dt, int64_t hidden, int64_t T);

}  // namespace dr

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------
#ifdef __HIPCC__
namespace dr {

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16 bytes of row data widened to fp32: 8 bf16 values or 4 fp32 values.
template <dr_dtype DT>
struct Vec;

template <>
struct Vec<DR_BF16> {
    static constexpr int kElems = 8;
    __device__ __forceinline__ static void widen(const u32x4& raw, float (&v)[8]) {
        v[0] = bf16_lo(raw.x); v[1] = bf16_hi(raw.x);
        v[2] = bf16_lo(raw.y); v[3] = bf16_hi(raw.y);
        v[4] = bf16_lo(raw.z); v[5] = bf16_hi(raw.z);
        v[6] = bf16_lo(raw.w); v[7] = bf16_hi(raw.w);
    }
};

template <>
struct Vec<DR_F32> {
    static constexpr int kElems = 4;
    __device__ __forceinline__ static void widen(const u32x4& raw, float (&v)[4]) {
        v[0] = __uint_as_float(raw.x); v[1] = __uint_as_float(raw.y);
        v[2] = __uint_as_float(raw.z); v[3] = __uint_as_float(raw.w);
    }
};

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// A lane's unit of row data: 4 consecutive columns, widened to fp32.  bf16
// rows are read as 8-byte pieces and fp32 rows as 16-byte pieces.  A lane owns
// kPieces pieces kSpan columns apart, so that both the loads and the 16-byte
// fp32 stores of a lane group cover contiguous bytes.
template <dr_dtype DT>
struct Piece;

template <>
struct Piece<DR_BF16> {
    static constexpr int kPieces = 2;
    typedef u32x2 Raw;
    __device__ __forceinline__ static Raw load(const void* row, int64_t col) {
        return *reinterpret_cast<const u32x2*>(reinterpret_cast<const uint16_t*>(row) + col);
    }
    __device__ __forceinline__ static Raw load_stream(const void* row, int64_t col) {
        return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(reinterpret_cast<const uint16_t*>(row) + col));
    }
    __device__ __forceinline__ static void widen(const Raw& r, float (&v)[4]) {
        v[0] = __uint_as_float(r.x << 16);
        v[1] = __uint_as_float(r.x & 0xFFFF0000u);
        v[2] = __uint_as_float(r.y << 16);
        v[3] = __uint_as_float(r.y & 0xFFFF0000u);
    }
};

template <>
struct Piece<DR_F32> {
    static constexpr int kPieces = 1;
    typedef u32x4 Raw;
    __device__ __forceinline__ static Raw load(const void* row, int64_t col) {
        return *reinterpret_cast<const u32x4*>(reinterpret_cast<const float*>(row) + col);
    }
    __device__ __forceinline__ static Raw load_stream(const void* row, int64_t col) {
        return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(reinterpret_cast<const float*>(row) + col));
    }
    __device__ __forceinline__ static void widen(const Raw& r, float (&v)[4]) {
        v[0] = __uint_as_float(r.x);
        v[1] = __uint_as_float(r.y);
        v[2] = __uint_as_float(r.z);
        v[3] = __uint_as_float(r.w);
    }
};

__device__ __forceinline__ u32x4 load16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ u32x4 load16_stream(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void store16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ void store16_stream(void* p, u32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// Column-strided access for the atomic baselines: lane l of a wavefront owns
// columns c0 + l + 64*e, so each memory or atomic instruction of the wavefront
// covers 64 consecutive elements (coalesced).
template <dr_dtype DT>
__device__ __forceinline__ float load_elem(const void* row, int64_t col) {
    if (DT == DR_BF16) return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(row)[col] << 16);
    return reinterpret_cast<const float*>(row)[col];
}

// The fingerprint's terms (see dr_fingerprint in detreduce.h): SplitMix64's
// finaliser (Steele, Lea and Flood, OOPSLA 2014) of a 64-bit word XOR the
// generator state (i + 1) * gamma.
__device__ __forceinline__ uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}
__device__ __forceinline__ uint64_t fp_term(uint64_t w, int64_t i) {
    return mix64(w ^ ((uint64_t)(i + 1) * 0x9e3779b97f4a7c15ull));
}
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int off) {
    const uint32_t lo = __shfl_xor((uint32_t)v, off, 64);
    const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), off, 64);
    return ((uint64_t)hi << 32) | lo;
}
// Wrapping sum over the workgroup (blockDim.x a multiple of 64, <= 1024); the
// result is valid in thread 0.  smem holds blockDim.x / 64 values.
__device__ __forceinline__ uint64_t block_sum_u64(uint64_t v, uint64_t* smem) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += shfl_xor_u64(v, off);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (lane == 0) smem[w] = v;
    __syncthreads();
    uint64_t s = 0;
    if (threadIdx.x == 0)
        for (int i = 0; i < (int)(blockDim.x >> 6); ++i) s += smem[i];
    return s;
}

// -0.0 is an exact identity of IEEE addition (x + -0.0 == x for every x,
// including +0.0 and -0.0), so padding a tree with it changes no bit.
__device__ __forceinline__ float neg_zero() { return __uint_as_float(0x80000000u); }

__device__ __forceinline__ uint64_t lanemask_lt() {
    return (uint64_t(1) << (threadIdx.x & 63)) - 1;
}

}  // namespace dr
#endif
