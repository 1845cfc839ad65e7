// index_add in the defined order: for each destination d, the rows of its
// contributions (in source order, from the sort) reduced by the fixed tree T,
// then out[d] = out[d] + T.
//
// The pages accumulate the many writers of a key row without atomics: the
// DeepSeek-V4 sparse-attention backward keeps per-SM partial key gradients and
// adds them in SM-id order (ch. 9, section 3.1).  That order depends on the
// number of SMs and needs a key-buffer slice per SM.  Here the partition is a
// property of the data instead: each destination's ordered contributions are
// cut into tiles of 2^m chunks of 8 rows, aligned at the segment start.  The
// tree splits only at aligned powers of two, so a tile's subtree sum is a
// node of the destination's tree whatever m is, and any grid, tile size or
// schedule gives the same bits.
//
//   plan_count / plan_write: tiles per destination, prefix sums, tile records.
//   segreduce:   one lane group per (tile, column slice), 16 bytes of each row
//                per lane.  It streams the tile's chunks (8 row loads in flight
//                per lane), sums each chunk left to right, and merges chunk
//                sums on a binary counter.
//                A destination with one tile is updated in place; the tiles of
//                a longer one write private partial rows.
//   tilecombine: merges a destination's partial rows by the same counter, in
//                tile order, then updates the destination row.
//   segreduce_gen16 / segreduce_gen: the formed-contribution form (the
//                sparse-attention key gradient), each row fl32(scale * a short
//                shared source row), one wavefront per tile.
#include "internal.h"
#include "lds_tile.h"

namespace dr {
namespace {

constexpr int kPlanThreads = 256;
constexpr int kPlanWaves = kPlanThreads / 64;
constexpr int kReduceThreads = 256;

struct TileCount {
    int32_t tiles;   // tiles of the segment
    int32_t multi;   // 1 if the segment has more than one tile
    int32_t pslots;  // partial slots the segment needs (its tile count when multi)
};

__device__ __forceinline__ TileCount tile_count(int32_t L, int tc_log2) {
    TileCount c{0, 0, 0};
    if (L > 0) {
        const int32_t chunks = (L + 7) >> 3;
        c.tiles = (chunks + (1 << tc_log2) - 1) >> tc_log2;
        c.multi = c.tiles > 1;
        c.pslots = c.multi ? c.tiles : 0;
    }
    return c;
}

__device__ __forceinline__ int32_t wave_sum(int32_t v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

__device__ __forceinline__ int32_t wave_inclusive_scan(int32_t v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int32_t t = __shfl_up(v, off, 64);
        if (lane >= off) v += t;
    }
    return v;
}

// Per destination: check the offsets, count tiles; per workgroup: the sums.
__global__ __launch_bounds__(kPlanThreads) void plan_count_kernel(const int32_t* __restrict__ seg, int32_t num_dests,
                                                                  int64_t n, int tc_log2, int32_t* block_sums,
                                                                  int32_t* status) {
    __shared__ int32_t part[3][kPlanWaves];
    if (status[kWordStatus] != 0) return;
    const int64_t d = (int64_t)blockIdx.x * kPlanThreads + threadIdx.x;
    TileCount c{0, 0, 0};
    bool bad = false;
    if (d < num_dests) {
        const int32_t a = seg[d], b = seg[d + 1];
        if (a < 0 || b < a || b > n) bad = true;
        else c = tile_count(b - a, tc_log2);
        if (d == 0 && a != 0) bad = true;
        if (d == num_dests - 1 && b != n) bad = true;
    }
    if (bad) atomicOr(&status[kWordStatus], kStatusPlan);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int32_t st = wave_sum(c.tiles), sm = wave_sum(c.multi), sp = wave_sum(c.pslots);
    if (lane == 0) {
        part[0][w] = st;
        part[1][w] = sm;
        part[2][w] = sp;
    }
    __syncthreads();
    if (threadIdx.x < 3) {
        int32_t s = 0;
        for (int i = 0; i < kPlanWaves; ++i) s += part[threadIdx.x][i];
        block_sums[3 * blockIdx.x + threadIdx.x] = s;
    }
}

// plan_count for a plan the library's own sort produced: thread d finds the
// lower bound of d in the sorted destinations (the workgroup's last thread
// also that of d + 1, in the same loop), first among 1024 evenly spaced
// samples held in LDS, then within one sample stride.  The next destination's
// bound comes from the neighbouring thread through LDS, and the thread writes
// the segment offset (the last destination's thread also seg[num_dests] = n)
// and counts tiles as plan_count does.  This replaces a separate offsets
// kernel.  The sort has already checked every destination, so there is
// nothing to validate.
__global__ __launch_bounds__(kPlanThreads) void plan_count_search_kernel(const int32_t* __restrict__ sorted_dest,
                                                                         int64_t n, int32_t num_dests, int tc_log2,
                                                                         int32_t* __restrict__ seg,
                                                                         int32_t* block_sums, int32_t* status) {
    constexpr int kSamples = 1024;  // every stride-th sorted destination, in LDS
    __shared__ int32_t part[3][kPlanWaves];
    __shared__ int32_t bound[kPlanThreads + 1];
    __shared__ int32_t sample[kSamples];
    if (status[kWordStatus] != 0) return;
    const int64_t d = (int64_t)blockIdx.x * kPlanThreads + threadIdx.x;
    const bool last = threadIdx.x == kPlanThreads - 1;
    const int64_t stride = (n + kSamples - 1) / kSamples;
    for (int k = threadIdx.x; k < kSamples; k += kPlanThreads)
        sample[k] = (int64_t)k * stride < n ? sorted_dest[(int64_t)k * stride] : INT32_MAX;
    __syncthreads();
    // The samples bound each search to one stride: with k the first sample
    // >= x, the lower bound of x lies in ((k-1)*stride, min(k*stride, n)].
    auto narrow = [&](int64_t x, int64_t& lo, int64_t& hi) {
        int a = 0, b = kSamples;  // first sample index with sample >= x
        while (a < b) {
            const int m = (a + b) >> 1;
            if (sample[m] < x) a = m + 1;
            else b = m;
        }
        lo = a == 0 ? 0 : (int64_t)(a - 1) * stride + 1;
        hi = min((int64_t)a * stride, n);
        if (lo > hi) lo = hi;
    };
    int64_t lo0 = n, hi0 = n, lo1 = 0, hi1 = 0;
    if (d <= num_dests) narrow(d, lo0, hi0);
    if (last && d < num_dests) narrow(d + 1, lo1, hi1);
    while (lo0 < hi0 || lo1 < hi1) {
        if (lo0 < hi0) {
            const int64_t mid = (lo0 + hi0) >> 1;
            if (sorted_dest[mid] < d) lo0 = mid + 1;
            else hi0 = mid;
        }
        if (lo1 < hi1) {
            const int64_t mid = (lo1 + hi1) >> 1;
            if (sorted_dest[mid] < d + 1) lo1 = mid + 1;
            else hi1 = mid;
        }
    }
    bound[threadIdx.x] = (int32_t)lo0;
    if (last) bound[kPlanThreads] = (int32_t)lo1;
    __syncthreads();
    TileCount c{0, 0, 0};
    if (d < num_dests) {
        const int32_t b = bound[threadIdx.x + 1];  // lower bound of d + 1
        seg[d] = (int32_t)lo0;
        if (d == num_dests - 1) seg[num_dests] = b;
        c = tile_count(b - (int32_t)lo0, tc_log2);
    }
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int32_t st = wave_sum(c.tiles), sm = wave_sum(c.multi), sp = wave_sum(c.pslots);
    if (lane == 0) {
        part[0][w] = st;
        part[1][w] = sm;
        part[2][w] = sp;
    }
    __syncthreads();
    if (threadIdx.x < 3) {
        int32_t t = 0;
        for (int i = 0; i < kPlanWaves; ++i) t += part[threadIdx.x][i];
        block_sums[3 * blockIdx.x + threadIdx.x] = t;
    }
}

// Exclusive prefix of the three counts over all destinations; writes one
// TileRec per tile and one MultiRec per destination with several tiles.
__global__ __launch_bounds__(kPlanThreads) void plan_write_kernel(const int32_t* __restrict__ seg, int32_t num_dests,
                                                                  int tc_log2, const int32_t* __restrict__ block_sums,
                                                                  TileRec* __restrict__ tiles,
                                                                  MultiRec* __restrict__ multis, int32_t* status) {
    __shared__ int32_t part[3][kPlanWaves];
    __shared__ int32_t base[3];
    if (status[kWordStatus] != 0) return;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    // sums of the earlier workgroups
    int32_t pt = 0, pm = 0, pp = 0;
    for (int64_t b = threadIdx.x; b < blockIdx.x; b += kPlanThreads) {
        pt += block_sums[3 * b];
        pm += block_sums[3 * b + 1];
        pp += block_sums[3 * b + 2];
    }
    pt = wave_sum(pt);
    pm = wave_sum(pm);
    pp = wave_sum(pp);
    if (lane == 0) {
        part[0][w] = pt;
        part[1][w] = pm;
        part[2][w] = pp;
    }
    __syncthreads();
    if (threadIdx.x < 3) {
        int32_t s = 0;
        for (int i = 0; i < kPlanWaves; ++i) s += part[threadIdx.x][i];
        base[threadIdx.x] = s;
    }
    __syncthreads();
    // own destinations
    const int64_t d = (int64_t)blockIdx.x * kPlanThreads + threadIdx.x;
    TileCount c{0, 0, 0};
    if (d < num_dests) c = tile_count(seg[d + 1] - seg[d], tc_log2);
    const int32_t it = wave_inclusive_scan(c.tiles), im = wave_inclusive_scan(c.multi),
                  ip = wave_inclusive_scan(c.pslots);
    __syncthreads();
    if (lane == 63) {
        part[0][w] = it;
        part[1][w] = im;
        part[2][w] = ip;
    }
    __syncthreads();
    int32_t wt = 0, wm = 0, wp = 0, tt = 0, tm = 0;
    for (int i = 0; i < kPlanWaves; ++i) {
        if (i < w) {
            wt += part[0][i];
            wm += part[1][i];
            wp += part[2][i];
        }
        tt += part[0][i];
        tm += part[1][i];
    }
    const int32_t tile0 = base[0] + wt + it - c.tiles;
    const int32_t multi0 = base[1] + wm + im - c.multi;
    const int32_t pslot0 = base[2] + wp + ip - c.pslots;
    for (int32_t j = 0; j < c.tiles; ++j) {
        TileRec r;
        r.dest = (int32_t)d;
        r.r_begin = seg[d] + ((j << tc_log2) << 3);
        r.r_end = (int32_t)min((int64_t)seg[d + 1], (int64_t)r.r_begin + (8 << tc_log2));  // no int32 overflow
        r.pslot = c.multi ? pslot0 + j : -1;
        tiles[tile0 + j] = r;
    }
    if (c.multi) {
        MultiRec m;
        m.dest = (int32_t)d;
        m.pslot0 = pslot0;
        m.ntiles = c.tiles;
        m.pad = 0;
        multis[multi0] = m;
    }
    if (blockIdx.x == gridDim.x - 1 && threadIdx.x == 0) {
        status[kWordTiles] = base[0] + tt;
        status[kWordMultis] = base[1] + tm;
    }
}

// Checks a caller-supplied plan: every sorted position r holds a source row
// p = perm[r] in range whose index[p] = d satisfies seg[d] <= r < seg[d+1],
// and the next position of the same segment holds a larger source row.  Then
// perm is injective (rows of different segments have different indices), so
// it is a permutation, each segment holds exactly its destination's rows, in
// ascending source order: the stable sort itself, and nothing else passes.
__global__ void plan_validate_kernel(const int32_t* __restrict__ perm, const int32_t* __restrict__ seg,
                                     const int32_t* __restrict__ index, int64_t n, int32_t num_dests,
                                     int32_t* status) {
    const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= n) return;
    const int32_t p = perm[r];
    int32_t err = 0;
    if (p < 0 || p >= n) {
        err = kStatusPlan;
    } else {
        const int32_t d = index[p];
        if (d < 0 || d >= num_dests) {
            err = kStatusIndex;
        } else {
            const int32_t lo = seg[d], hi = seg[d + 1];
            if (r < lo || r >= hi) err = kStatusPlan;
            else if (r + 1 < hi && r + 1 < n && perm[r + 1] <= p) err = kStatusPlan;  // source order
        }
    }
    if (err) atomicOr(&status[kWordStatus], err);
}

// Binary counter of subtree sums: level l holds a complete subtree of 2^l
// leaves.  push() merges the new leaf with the filled levels below the first
// empty one (left operand first) and stores it there; fold() combines the
// remaining subtrees from the right.  This gives T for any leaf count.  Level
// indices are compile-time, which keeps the levels in registers.  When the
// count is the same in the whole wavefront (UNIFORM: one lane group per
// wavefront), a level's additions run under a wave-uniform branch, so a push
// or fold adds only at the levels it touches; otherwise every level is
// computed and selected.  Stores into the levels stay selects either way.
// Both forms perform the same additions in the same order.
template <int DEPTH, int E, bool UNIFORM = false>
struct TreeCounter {
    float level[DEPTH][E];
    uint32_t count = 0;

    __device__ __forceinline__ TreeCounter() {
#pragma unroll
        for (int l = 0; l < DEPTH; ++l) {
#pragma unroll
            for (int e = 0; e < E; ++e) level[l][e] = neg_zero();
        }
    }

    __device__ __forceinline__ void push(float (&s)[E]) {
        if (UNIFORM) {
            // (the empty asm statement keeps the compiler from turning the
            // wave-uniform merge branches into per-lane selects over every level)
            const int merges = __builtin_amdgcn_readfirstlane(__builtin_ctz(~count));
#pragma unroll
            for (int l = 0; l < DEPTH; ++l) {
                if (l < merges) {
                    asm volatile("");
#pragma unroll
                    for (int e = 0; e < E; ++e) s[e] = level[l][e] + s[e];
                }
            }
#pragma unroll
            for (int l = 0; l < DEPTH; ++l) {
#pragma unroll
                for (int e = 0; e < E; ++e) level[l][e] = l == merges ? s[e] : level[l][e];
            }
            ++count;
            return;
        }
        const int merges = __builtin_ctz(~count);  // carries of this increment
#pragma unroll
        for (int l = 0; l < DEPTH; ++l) {
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float a = level[l][e] + s[e];
                s[e] = l < merges ? a : s[e];
            }
        }
#pragma unroll
        for (int l = 0; l < DEPTH; ++l) {
#pragma unroll
            for (int e = 0; e < E; ++e) level[l][e] = l == merges ? s[e] : level[l][e];
        }
        ++count;
    }

    __device__ __forceinline__ void fold(float (&acc)[E]) const {
        bool have = false;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] = neg_zero();
        if (UNIFORM) {
            const uint32_t c = __builtin_amdgcn_readfirstlane(count);
#pragma unroll
            for (int l = 0; l < DEPTH; ++l) {
                if ((c >> l) & 1u) {
#pragma unroll
                    for (int e = 0; e < E; ++e) acc[e] = have ? level[l][e] + acc[e] : level[l][e];
                    have = true;
                }
            }
            return;
        }
#pragma unroll
        for (int l = 0; l < DEPTH; ++l) {
            const bool bit = (count >> l) & 1u;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float a = level[l][e] + acc[e];
                acc[e] = bit ? (have ? a : level[l][e]) : acc[e];
            }
            have = have || bit;
        }
    }
};

// The binary counter for a count that is the same in the whole wavefront
// (one lane group per wavefront), with the same additions in the same order
// as TreeCounter.  A push merges under wave-uniform branches, and its one
// store goes to the level the carries end at: a wave-uniform index into a
// register vector (relative VGPR addressing: one move per element, where a
// store into an array of levels is a select at every level).  A vector of 16
// holds the levels of two elements up to depth 8, of one up to 16; deeper
// counters take a vector of 32 per element.
template <int DEPTH, int E>
struct UniformTreeCounter {
    static_assert(DEPTH <= 32, "levels");
    static constexpr int kPer = DEPTH <= 8 ? 8 : (DEPTH <= 16 ? 16 : 32);  // slots per element
    static constexpr int kW = kPer <= 16 ? 16 : 32;                         // vector width
    static constexpr int kEpv = kW / kPer;                                  // elements per vector
    typedef float lv_t __attribute__((ext_vector_type(kW)));
    lv_t lev[(E + kEpv - 1) / kEpv];  // level l of element e: lev[e / kEpv][kPer (e % kEpv) + l]
    uint32_t count = 0;

    __device__ __forceinline__ UniformTreeCounter() {
#pragma unroll
        for (int e = 0; e < E; ++e) {
#pragma unroll
            for (int l = 0; l < DEPTH; ++l) lev[e / kEpv][kPer * (e % kEpv) + l] = neg_zero();
        }
    }

    __device__ __forceinline__ void push(float (&s)[E]) {
        // (the empty asm statement keeps the merge branches from becoming
        // per-lane selects over every level)
        const int merges = __builtin_amdgcn_readfirstlane(__builtin_ctz(~count));
#pragma unroll
        for (int l = 0; l < DEPTH; ++l) {
            if (l < merges) {
                asm volatile("");
#pragma unroll
                for (int e = 0; e < E; ++e) s[e] = lev[e / kEpv][kPer * (e % kEpv) + l] + s[e];
            }
        }
        // the count stays below 2^DEPTH - 1 (the host sizes DEPTH), so merges < DEPTH
#pragma unroll
        for (int e = 0; e < E; ++e) lev[e / kEpv][kPer * (e % kEpv) + merges] = s[e];
        ++count;
    }

    __device__ __forceinline__ void fold(float (&acc)[E]) const {
        bool have = false;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] = neg_zero();
        const uint32_t c = __builtin_amdgcn_readfirstlane(count);
#pragma unroll
        for (int l = 0; l < DEPTH; ++l) {
            if ((c >> l) & 1u) {
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const float v = lev[e / kEpv][kPer * (e % kEpv) + l];
                    acc[e] = have ? v + acc[e] : v;
                }
                have = true;
            }
        }
    }
};

__device__ __forceinline__ u32x4 add4(const u32x4& old, const float* t) {
    // out = old + T: the old value is the left operand, added once, last
    u32x4 r;
    r.x = __float_as_uint(__uint_as_float(old.x) + t[0]);
    r.y = __float_as_uint(__uint_as_float(old.y) + t[1]);
    r.z = __float_as_uint(__uint_as_float(old.z) + t[2]);
    r.w = __float_as_uint(__uint_as_float(old.w) + t[3]);
    return r;
}

// Change of the fingerprint terms of one 16-byte piece of the destination
// (two 8-byte words starting at word index i) when old becomes now: the
// fingerprint is a wrapping sum of position-keyed word terms, so rewriting
// the piece adds exactly this to it.
__device__ __forceinline__ uint64_t fp_delta(const u32x4& old, const u32x4& now, int64_t i) {
    const uint64_t o0 = ((uint64_t)old.y << 32) | old.x, o1 = ((uint64_t)old.w << 32) | old.z;
    const uint64_t n0 = ((uint64_t)now.y << 32) | now.x, n1 = ((uint64_t)now.w << 32) | now.z;
    return (fp_term(n0, i) + fp_term(n1, i + 1)) - (fp_term(o0, i) + fp_term(o1, i + 1));
}

__device__ __forceinline__ u32x4 pack4(const float* t) {
    return u32x4{__float_as_uint(t[0]), __float_as_uint(t[1]), __float_as_uint(t[2]), __float_as_uint(t[3])};
}

// Lane groups of GROUP lanes; each lane owns 16 consecutive bytes of a row (8
// bf16 or 4 fp32 columns), so every row load is one 16-byte load per lane and
// a group reads GROUP*16 contiguous bytes.  One group reduces one (tile,
// column slice).
//
// Four wavefronts per SIMD (at most 128 VGPRs) for one item per wavefront with
// tiles of up to 2^5 chunks; deeper counters would spill at that budget.
template <dr_dtype DT, int GROUP, int TCLOG, int CIF>
__global__ __launch_bounds__(kReduceThreads, GROUP == 64 && CIF == 1 && TCLOG <= 5 ? 4 : 1) void segreduce_kernel(
    float* __restrict__ out, int64_t H, const void* __restrict__ src, const int32_t* __restrict__ perm,
    const TileRec* __restrict__ tiles, float* __restrict__ partials, int64_t slices, int32_t* status,
    uint64_t* __restrict__ fp_part) {
    using V = Vec<DT>;
    constexpr int E = V::kElems;  // columns of a lane
    constexpr int Q = E / 4;      // 16-byte fp32 pieces of a lane's output
    constexpr int kElemBytes = DT == DR_BF16 ? 2 : 4;
    constexpr int64_t W = (int64_t)GROUP * E;  // columns of one group slice
    if (status[kWordStatus] != 0) return;
    // the host keeps (tile bound) * slices below 2^32, so 32-bit division suffices
    const uint32_t items = (uint32_t)status[kWordTiles] * (uint32_t)slices;
    const int lig = threadIdx.x % GROUP;
    uint32_t group = (blockIdx.x * kReduceThreads + threadIdx.x) / GROUP;
    if (GROUP == 64) group = __builtin_amdgcn_readfirstlane(group);  // one item per wavefront
    const uint32_t ngroups = (gridDim.x * kReduceThreads) / GROUP;
    const char* src_bytes = reinterpret_cast<const char*>(src);
    const int64_t row_bytes = H * kElemBytes;
    uint64_t fp_acc = 0;  // change of the destination's fingerprint made by this lane
    // With one item per wavefront (AHEAD), tile records are fetched two items
    // ahead and the source ids of an item's first rows while the previous
    // item's last rows arrive, so an item starts with its row loads (the item
    // index is wave-uniform, so the records sit in scalar registers).
    // Otherwise the record is fetched one item ahead and the first ids at the
    // item's start, which keeps the lane groups' registers within three
    // wavefronts per SIMD.
    constexpr bool AHEAD = GROUP == 64;
    constexpr int R = 8 * CIF;  // rows loaded at once (CIF chunks of 8)
    TileRec tr_next{}, tr_next2{};
    int32_t idx[R];
    if (group < items) {
        tr_next = tiles[group / (uint32_t)slices];
        if (AHEAD) {
#pragma unroll
            for (int j = 0; j < R; ++j) idx[j] = perm[min(tr_next.r_begin + j, tr_next.r_end - 1)];
        }
    }
    if (AHEAD && (uint64_t)group + ngroups < items) tr_next2 = tiles[(group + ngroups) / (uint32_t)slices];
    for (uint32_t it = group; it < items; it += ngroups) {
        const uint32_t tile = it / (uint32_t)slices;
        const uint32_t slice = it - tile * (uint32_t)slices;
        const TileRec tr = tr_next;
        const bool has_next = (uint64_t)it + ngroups < items;
        if (AHEAD) {
            tr_next = tr_next2;
            if ((uint64_t)it + 2ull * ngroups < items) tr_next2 = tiles[(it + 2 * ngroups) / (uint32_t)slices];
        } else if (has_next) {
            tr_next = tiles[(it + ngroups) / (uint32_t)slices];
        }
        const int64_t col = (int64_t)slice * W + E * lig;
        const bool active = col < H;
        const int64_t lcol = active ? col : 0;  // idle lanes read a valid piece
        const int64_t r_begin = tr.r_begin, r_end = tr.r_end;
        float* orow = out + (int64_t)tr.dest * H;
        // the destination row, fetched early when this tile updates it in place
        u32x4 old[Q];
        if (tr.pslot < 0) {
#pragma unroll
            for (int q = 0; q < Q; ++q) old[q] = load16(orow + lcol + 4 * q);
        }
        TreeCounter<TCLOG + 1, E, GROUP == 64> tc;
        // CIF chunks (8*CIF rows) are loaded at once; slots past the tile's
        // end are neither loaded nor added.
        if (!AHEAD) {
#pragma unroll
            for (int j = 0; j < R; ++j) idx[j] = perm[min(r_begin + j, r_end - 1)];
        }
        for (int64_t r0 = r_begin; r0 < r_end; r0 += R) {
            u32x4 raw[R];
            const int64_t live = r_end - r0;  // rows of this step that exist
            if (live >= R) {
#pragma unroll
                for (int j = 0; j < R; ++j)
                    raw[j] = load16_stream(src_bytes + (int64_t)idx[j] * row_bytes + lcol * kElemBytes);
            } else {
#pragma unroll
                for (int j = 0; j < R; ++j) {
                    raw[j] = u32x4{0u, 0u, 0u, 0u};
                    if (j < live) raw[j] = load16_stream(src_bytes + (int64_t)idx[j] * row_bytes + lcol * kElemBytes);
                }
            }
            // the next rows' source ids (this item's, else the next item's
            // first) are fetched while these rows arrive
            const int64_t r1 = r0 + R;
            if (r1 < r_end) {
#pragma unroll
                for (int j = 0; j < R; ++j) idx[j] = perm[min(r1 + j, r_end - 1)];
            } else if (AHEAD && has_next) {
#pragma unroll
                for (int j = 0; j < R; ++j) idx[j] = perm[min(tr_next.r_begin + j, tr_next.r_end - 1)];
            }
#pragma unroll
            for (int c = 0; c < CIF; ++c) {
                int m = (int)min((int64_t)8, r_end - (r0 + 8 * c));  // rows of chunk c (<= 0: none)
                if (GROUP == 64) m = __builtin_amdgcn_readfirstlane(m);  // one tile per wavefront
                if (m > 0) {
                    float s[E];
                    V::widen(raw[8 * c], s);
                    if (m == 8) {
#pragma unroll
                        for (int j = 1; j < 8; ++j) {
                            float v[E];
                            V::widen(raw[8 * c + j], v);
#pragma unroll
                            for (int e = 0; e < E; ++e) s[e] = s[e] + v[e];
                        }
                    } else if (GROUP == 64) {
                        // wave-uniform row count: the rows past it are skipped, not computed
#pragma unroll
                        for (int j = 1; j < 8; ++j) {
                            if (j < m) {
                                float v[E];
                                V::widen(raw[8 * c + j], v);
#pragma unroll
                                for (int e = 0; e < E; ++e) s[e] = s[e] + v[e];
                            }
                        }
                    } else {
#pragma unroll
                        for (int j = 1; j < 8; ++j) {
                            float v[E];
                            V::widen(raw[8 * c + j], v);
#pragma unroll
                            for (int e = 0; e < E; ++e) {
                                const float a = s[e] + v[e];
                                s[e] = j < m ? a : s[e];
                            }
                        }
                    }
                    tc.push(s);
                }
            }
        }
        float t[E];
        tc.fold(t);
        if (active) {
            if (tr.pslot < 0) {
#pragma unroll
                for (int q = 0; q < Q; ++q) {
                    const u32x4 now = add4(old[q], t + 4 * q);
                    store16(orow + col + 4 * q, now);
                    if (fp_part) fp_acc += fp_delta(old[q], now, ((int64_t)tr.dest * H + col + 4 * q) >> 1);
                }
            } else {
                float* prow = partials + (int64_t)tr.pslot * H;
#pragma unroll
                for (int q = 0; q < Q; ++q) store16(prow + col + 4 * q, pack4(t + 4 * q));
            }
        }
    }
    if (fp_part) {
        __shared__ uint64_t fsm[kReduceThreads / 64];
        const uint64_t b = block_sum_u64(fp_acc, fsm);
        if (threadIdx.x == 0) fp_part[blockIdx.x] = b;
    }
}

// The formed-contribution reduce (the sparse-attention key gradient): the
// contribution of sorted position r, source row p = perm[r], is
// fl32(scale * src[p / rows_per_src]) element by element, with scale the
// score gradient of that row (scale[r] when the sort moved the scales into
// sorted order, else scale[p]).  One wavefront per (tile, column slice), lane
// l owning E consecutive columns, so that a short source row (128 columns)
// still fills the wavefront and every row step is wave-uniform: lanes 0..7
// fetch a chunk's ids and scales and the row loads read them back with
// readlane, each row is one small load per lane (the source rows are few and
// shared, so they are read through the cache), and the chunk sums and the
// tree need no per-lane selects.  This form serves fp32 source rows and
// sources of 2^31 bytes or 2^24 rows or more; bf16 rows take the LDS form
// below.  The arithmetic
// is the same as the row kernel's: chunks of 8 rows left to right, the chunk
// sums into the pairwise tree, the tile's result added once into the
// destination row (or stored as the tile's partial row for tilecombine).
template <dr_dtype DT, int E>
struct GenRow {
    static constexpr int kBytes = E * (DT == DR_BF16 ? 2 : 4);
    static constexpr int kWords = kBytes / 4;
    typedef uint32_t Raw __attribute__((ext_vector_type(kWords)));
    __device__ __forceinline__ static Raw load(const char* p) { return *reinterpret_cast<const Raw*>(p); }
    __device__ __forceinline__ static void widen(const Raw& r, float (&v)[E]) {
#pragma unroll
        for (int w = 0; w < kWords; ++w) {
            if (DT == DR_BF16) {
                v[2 * w] = __uint_as_float(r[w] << 16);
                v[2 * w + 1] = __uint_as_float(r[w] & 0xFFFF0000u);
            } else {
                v[w] = __uint_as_float(r[w]);
            }
        }
    }
};

#ifndef GEN_CHUNKS
#define GEN_CHUNKS 2
#endif
// Source row of contribution p: p / rows_per_src as (p * m) >> (31 + sh), with
// m = ceil(2^(31+sh) / d) and sh = ceil(log2 d): exact for p < 2^31 (the error
// of m, below d, moves p * m / 2^(31+sh) by less than 2^-sh <= 1/d).
__device__ __forceinline__ uint32_t gen_row_of(uint32_t p, uint32_t m, uint32_t sh) {
    return (uint32_t)(((uint64_t)p * m) >> (31 + sh));
}

template <dr_dtype DT, int E, int TCLOG, bool SORTED>
__global__ __launch_bounds__(kReduceThreads) void segreduce_gen_kernel(
    float* __restrict__ out, int64_t H, const char* __restrict__ src, const int32_t* __restrict__ perm,
    const TileRec* __restrict__ tiles, float* __restrict__ partials, int64_t slices, const int32_t* __restrict__ status,
    const float* __restrict__ scale, uint32_t div_m, uint32_t div_sh) {
    using G = GenRow<DT, E>;
    constexpr int kElemBytes = DT == DR_BF16 ? 2 : 4;
    constexpr int CH = GEN_CHUNKS;  // chunks of 8 rows loaded at once
    constexpr int R = 8 * CH;
    if (status[kWordStatus] != 0) return;
    // the host keeps (tile bound) * slices below 2^32, so 32-bit division suffices
    const uint32_t items = (uint32_t)status[kWordTiles] * (uint32_t)slices;
    const int lane = threadIdx.x & 63;
    const uint32_t wave = __builtin_amdgcn_readfirstlane((blockIdx.x * kReduceThreads + threadIdx.x) / 64);
    const uint32_t nwaves = gridDim.x * (kReduceThreads / 64);
    const int64_t row_bytes = H * kElemBytes;
    const int jl = lane % R;
    // Lanes 0..R-1 hold the source ids of the next R rows (rows past a tile's
    // end repeat its last row and are not added), fetched one step ahead: the
    // next item's first ids are fetched during the current item's last step.
    TileRec tr_next{};
    int32_t ids = 0;
    if (wave < items) {
        tr_next = tiles[wave / (uint32_t)slices];
        ids = perm[min((int64_t)tr_next.r_begin + jl, (int64_t)tr_next.r_end - 1)];
    }
    for (uint32_t it = wave; it < items; it += nwaves) {
        const uint32_t slice = it % (uint32_t)slices;
        const TileRec tr = tr_next;
        const bool has_next = (uint64_t)it + nwaves < items;
        if (has_next) tr_next = tiles[(it + nwaves) / (uint32_t)slices];
        const int64_t col = (int64_t)slice * 64 * E + E * lane;
        const bool active = col < H;
        const int64_t lcol = active ? col : 0;  // idle lanes read a valid piece
        const char* src_col = src + lcol * kElemBytes;
        const int64_t r_begin = tr.r_begin, r_end = tr.r_end;
        float* orow = out + (int64_t)tr.dest * H;
        float old[E];
        if (tr.pslot < 0) {
#pragma unroll
            for (int e = 0; e < E; ++e) old[e] = orow[lcol + e];
        }
        TreeCounter<TCLOG + 1, E, true> tc;
        for (int64_t r0 = r_begin; r0 < r_end; r0 += R) {
            const float scl = scale[SORTED ? min(r0 + jl, r_end - 1) : (int64_t)ids];
            typename G::Raw raw[R];
#pragma unroll
            for (int j = 0; j < R; ++j) {
                const uint32_t p = (uint32_t)__builtin_amdgcn_readlane(ids, j);
                raw[j] = G::load(src_col + (int64_t)gen_row_of(p, div_m, div_sh) * row_bytes);
            }
            const int64_t r1 = r0 + R;
            if (r1 < r_end) ids = perm[min(r1 + jl, r_end - 1)];
            else if (has_next) ids = perm[min((int64_t)tr_next.r_begin + jl, (int64_t)tr_next.r_end - 1)];
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                const int m = (int)min((int64_t)8, r_end - (r0 + 8 * c));  // rows of chunk c (wave-uniform)
                if (m > 0) {
                    float s[E];
                    G::widen(raw[8 * c], s);
                    const float s0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                                 __builtin_bit_cast(int32_t, scl), 8 * c));
#pragma unroll
                    for (int e = 0; e < E; ++e) s[e] = s0 * s[e];
#pragma unroll
                    for (int j = 1; j < 8; ++j) {
                        if (j < m) {
                            const float sj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                                         __builtin_bit_cast(int32_t, scl), 8 * c + j));
                            float v[E];
                            G::widen(raw[8 * c + j], v);
#pragma unroll
                            for (int e = 0; e < E; ++e) v[e] = sj * v[e];  // rounded product
#pragma unroll
                            for (int e = 0; e < E; ++e) s[e] = s[e] + v[e];
                        }
                    }
                    tc.push(s);
                }
            }
        }
        float t[E];
        tc.fold(t);
        if (active) {
            if (tr.pslot < 0) {
#pragma unroll
                for (int e = 0; e < E; ++e) orow[col + e] = old[e] + t[e];  // out = old + T
            } else {
                float* prow = partials + (int64_t)tr.pslot * H;
#pragma unroll
                for (int e = 0; e < E; ++e) prow[col + e] = t[e];
            }
        }
    }
}

// The formed-contribution reduce for bf16 source rows, through LDS.  Row
// loads are 16 bytes per lane (a 16-lane group reads one 128-column slice of a
// row, four rows per instruction: 16-byte loads move four times the bytes of
// the 4-byte loads above for the same address work); the wavefront writes a
// chunk's 8 rows to its own 2 KB of LDS and reads them back transposed with
// ds_read_b64_tr_b16, so that lane l holds columns l and 64 + l of all 8 rows
// and the chunk sum, the tree and the destination update run wave-uniform, as
// above.  Each lane group fetches the ids of its two rows of a chunk with one
// 8-byte vector load, one chunk ahead (so a chunk waits for its rows only),
// and forms their byte offsets with two 24-bit multiply-adds (the host keeps
// source rows and row bytes below 2^24); the chunk's 8 scales arrive in scalar
// registers by one 8-dword scalar buffer load (sorted scales; else the ids
// come the same way and the scales are fetched by id through the scalar
// cache).  The LDS tile is row-major with the
// 16-byte chunks of row r swizzled by r & 3, so a transposing read's four rows
// fall in different banks.
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));
typedef int32_t i32x8_t __attribute__((ext_vector_type(8)));
// Eight consecutive dwords through the scalar cache, range-checked: a dword at
// or past the resource's size reads as 0.
__device__ i32x8_t dr_s_buffer_load_x8(i32x4_t rsrc, int32_t offset, int32_t cachepolicy)
    __asm("llvm.amdgcn.s.buffer.load.v8i32");

__device__ __forceinline__ i32x4_t dword_rsrc(const void* p, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    return i32x4_t{(int32_t)(uint32_t)a, (int32_t)(uint32_t)(a >> 32), (int32_t)bytes, 0x00020000};
}

template <int TCLOG, bool SORTED, bool POW2>
__global__ __launch_bounds__(kReduceThreads) void segreduce_gen16_kernel(
    float* __restrict__ out, int64_t H, const char* __restrict__ src, uint32_t src_bytes,
    const int32_t* __restrict__ perm, uint32_t n, const TileRec* __restrict__ tiles, float* __restrict__ partials,
    int64_t slices, const int32_t* __restrict__ status, const float* __restrict__ scale, uint32_t div_m,
    uint32_t div_sh) {
    constexpr int kCols = 128;  // columns of a slice
    __shared__ __attribute__((aligned(16))) uint16_t lds_rows[kReduceThreads / 64][8 * kCols];
    if (status[kWordStatus] != 0) return;
    // the host keeps (tile bound) * slices below 2^32, so 32-bit division suffices
    const uint32_t items = (uint32_t)status[kWordTiles] * (uint32_t)slices;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int g = lane >> 4, li = lane & 15;  // loads: group g reads rows 2g and 2g + 1, 16-byte piece li
    const uint32_t wave = __builtin_amdgcn_readfirstlane((blockIdx.x * kReduceThreads + threadIdx.x) / 64);
    const uint32_t nwaves = gridDim.x * (kReduceThreads / 64);
    if (wave >= items) return;
    const uint32_t nsl = (uint32_t)slices;
    const uint32_t row_bytes = (uint32_t)H * 2;  // the host keeps the source rows below 2^31 bytes
    // source rows, ids and sorted scales through buffer resources (32-bit offsets)
    const __amdgpu_buffer_rsrc_t srsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(src), 0, (int)src_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t pvrsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t*>(perm), 0, (int)(4 * n), 0x00020000);
    const i32x4_t prsrc = dword_rsrc(perm, 4 * n);
    const i32x4_t crsrc = dword_rsrc(scale, 4 * n);
    uint16_t* rows = lds_rows[wv];
    // LDS offsets: this lane's two row writes, and its transposing reads (read k
    // covers rows 4 (k >> 1) .. + 3 of column block g + 4 (k & 1); lane (g, b, c)
    // addresses row 4 (k >> 1) + b, columns 16 (g + 4 (k & 1)) + 4 c).
    const int w0 = lds_at<kCols>(2 * g, 8 * li), w1 = lds_at<kCols>(2 * g + 1, 8 * li);
    int rd[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
        rd[k] = lds_at<kCols>(4 * (k >> 1) + ((lane >> 2) & 3), 16 * (g + 4 * (k & 1)) + 4 * (lane & 3));
    typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
    // this group's two ids (rows 2g and 2g + 1 of the chunk at r0) by one vector
    // load; rows past a tile's end (other tiles' rows, or 0 past the array's
    // end: the buffer loads check each dword against the size) are loaded but
    // not added
    auto load_ids = [&](int32_t r0) {
        return __builtin_bit_cast(u32x2v, __builtin_amdgcn_raw_buffer_load_b64(pvrsrc, 4 * (r0 + 2 * g), 0, 0));
    };
    auto tile_of = [&](uint32_t it) { return nsl == 1 ? it : it / nsl; };
    // The ids of each chunk are fetched one chunk ahead (the next item's first
    // ones during the current item's last chunk), and the next item's tile
    // record one item ahead, so a chunk waits for its rows only.
    TileRec tr = tiles[tile_of(wave)];
    TileRec trn{0, 0, 0, -1};
    if ((uint64_t)wave + nwaves < items) trn = tiles[tile_of(wave + nwaves)];
    u32x2v idv = load_ids(tr.r_begin);
    for (uint32_t it = wave; it < items; it += nwaves) {
        const uint32_t tile = tile_of(it);
        const int32_t c0 = (int32_t)(it - tile * nsl) * kCols;
        // loads: 8 columns from c0 + 8 li (idle pieces past H read the slice's first piece)
        const uint32_t lcol_off = (uint32_t)(c0 + 8 * li < H ? c0 + 8 * li : c0) * 2;
        const int32_t r_begin = tr.r_begin, r_end = tr.r_end;
        float* orow = out + (int64_t)tr.dest * H;
        const int32_t pslot = tr.pslot;
        // results: lane l owns columns c0 + l and c0 + 64 + l
        const int64_t oc0 = c0 + lane, oc1 = c0 + 64 + lane;
        const bool act0 = oc0 < H, act1 = oc1 < H;
        float old0 = 0.f, old1 = 0.f;
        if (pslot < 0) {
            old0 = orow[act0 ? oc0 : 0];
            old1 = orow[act1 ? oc1 : 0];
        }
        UniformTreeCounter<TCLOG + 1, 2> tc;
        for (int32_t r0 = r_begin; r0 < r_end; r0 += 8) {
            const int m = min(8, r_end - r0);  // rows of the chunk (wave-uniform)
            // source rows are below 2^24 and rows below 2^24 bytes (the host
            // checks), so 24-bit multiplies give the byte offsets
            const uint32_t ra = POW2 ? idv[0] >> div_sh : gen_row_of(idv[0], div_m, div_sh);
            const uint32_t rb = POW2 ? idv[1] >> div_sh : gen_row_of(idv[1], div_m, div_sh);
            const uint32_t oa = (uint32_t)__umul24(ra, row_bytes), ob = (uint32_t)__umul24(rb, row_bytes);
            const u32x4 va = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(srsrc, (int)(oa + lcol_off), 0, 0));
            const u32x4 vb = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(srsrc, (int)(ob + lcol_off), 0, 0));
            // the next chunk's ids: this tile's next chunk, else the next item's first
            const u32x2v idn = load_ids(r0 + 8 < r_end ? r0 + 8 : trn.r_begin);
            // the chunk's scales, wave-uniform
            float sc[8];
            if (SORTED) {
                const i32x8_t sv = dr_s_buffer_load_x8(crsrc, 4 * r0, 0);
#pragma unroll
                for (int j = 0; j < 8; ++j) sc[j] = __int_as_float(sv[j]);  // (not a bit_cast of the element lvalue)
            } else {
                const i32x8_t pv = dr_s_buffer_load_x8(prsrc, 4 * r0, 0);
#pragma unroll
                for (int j = 0; j < 8; ++j) sc[j] = scale[(uint32_t)pv[j]];
            }
            *reinterpret_cast<u32x4*>(rows + w0) = va;
            *reinterpret_cast<u32x4*>(rows + w1) = vb;
            __builtin_amdgcn_wave_barrier();
            typedef short s16x4 __attribute__((ext_vector_type(4)));
            typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
            s16x4 t[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) t[k] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(rows + rd[k]));
            __builtin_amdgcn_wave_barrier();
            // row j of column l: t[2 (j >> 2)][j & 3]; of column 64 + l: t[2 (j >> 2) + 1][j & 3]
            float s2[2];
            s2[0] = sc[0] * __uint_as_float((uint32_t)(uint16_t)t[0][0] << 16);
            s2[1] = sc[0] * __uint_as_float((uint32_t)(uint16_t)t[1][0] << 16);
#pragma unroll
            for (int j = 1; j < 8; ++j) {
                if (j < m) {
                    const float v0 = sc[j] * __uint_as_float((uint32_t)(uint16_t)t[(j >> 2) * 2][j & 3] << 16);
                    const float v1 = sc[j] * __uint_as_float((uint32_t)(uint16_t)t[(j >> 2) * 2 + 1][j & 3] << 16);
                    s2[0] = s2[0] + v0;  // rounded products, added left to right
                    s2[1] = s2[1] + v1;
                }
            }
            tc.push(s2);
            idv = idn;
        }
        float t2[2];
        tc.fold(t2);
        if (pslot < 0) {
            if (act0) orow[oc0] = old0 + t2[0];  // out = old + T
            if (act1) orow[oc1] = old1 + t2[1];
        } else {
            float* prow = partials + (int64_t)pslot * H;
            if (act0) prow[oc0] = t2[0];
            if (act1) prow[oc1] = t2[1];
        }
        tr = trn;
        if ((uint64_t)it + 2 * (uint64_t)nwaves < items) trn = tiles[tile_of(it + 2 * nwaves)];
    }
}

// Merges the partial rows of each multi-tile destination in tile order (the
// tiles are the leaves of the destination's tree at this level).  One
// wavefront per (destination, 128-column slice), lane l owning columns 2l and
// 2l + 1 of the slice (one 8-byte piece), so the tile count and the counter
// are the same in the whole wavefront; up to 16 partial rows are in flight
// per lane.
template <int DEPTH>
__global__ __launch_bounds__(kReduceThreads) void tilecombine_kernel(float* __restrict__ out, int64_t H,
                                                                     const float* __restrict__ partials,
                                                                     const MultiRec* __restrict__ multis,
                                                                     int64_t slices, int32_t* status,
                                                                     uint64_t* __restrict__ fp_part) {
    if (status[kWordStatus] != 0) return;
    constexpr int R = 16;  // partial rows in flight
    uint64_t fp_acc = 0;
    const uint32_t items = (uint32_t)status[kWordMultis] * (uint32_t)slices;
    const int lane = threadIdx.x & 63;
    const uint32_t wave = __builtin_amdgcn_readfirstlane((blockIdx.x * kReduceThreads + threadIdx.x) / 64);
    const uint32_t nwaves = gridDim.x * (kReduceThreads / 64);
    for (uint32_t it = wave; it < items; it += nwaves) {
        const uint32_t mi = it / (uint32_t)slices;
        const uint32_t slice = it - mi * (uint32_t)slices;
        const MultiRec mr = multis[mi];
        const int64_t col = (int64_t)slice * 128 + 2 * lane;
        const bool active = col < H;
        const int64_t lcol = active ? col : 0;  // idle lanes read a valid piece
        float* orow = out + (int64_t)mr.dest * H;
        const u32x2 old = *reinterpret_cast<const u32x2*>(orow + lcol);
        UniformTreeCounter<DEPTH, 2> tc;
        for (int32_t q0 = 0; q0 < mr.ntiles; q0 += R) {
            const int m = min(R, mr.ntiles - q0);  // wave-uniform
            u32x2 raw[R];
#pragma unroll
            for (int j = 0; j < R; ++j)
                raw[j] = *reinterpret_cast<const u32x2*>(partials + (int64_t)(mr.pslot0 + q0 + min(j, m - 1)) * H +
                                                         lcol);
#pragma unroll
            for (int j = 0; j < R; ++j) {
                if (j < m) {
                    float v[2] = {__uint_as_float(raw[j].x), __uint_as_float(raw[j].y)};
                    tc.push(v);
                }
            }
        }
        float t[2];
        tc.fold(t);
        // out = old + T: the old value is the left operand, added once, last
        const u32x2 now{__float_as_uint(__uint_as_float(old.x) + t[0]), __float_as_uint(__uint_as_float(old.y) + t[1])};
        if (active) {
            *reinterpret_cast<u32x2*>(orow + col) = now;
            if (fp_part) {
                const int64_t w = ((int64_t)mr.dest * H + col) >> 1;
                fp_acc += fp_term(((uint64_t)now.y << 32) | now.x, w) - fp_term(((uint64_t)old.y << 32) | old.x, w);
            }
        }
    }
    if (fp_part) {
        __shared__ uint64_t fsm[kReduceThreads / 64];
        const uint64_t b = block_sum_u64(fp_acc, fsm);
        if (threadIdx.x == 0) fp_part[blockIdx.x] = b;
    }
}

int group_for(int64_t pieces) {
    if (pieces <= 16) return 16;
    if (pieces <= 32) return 32;
    return 64;
}

template <dr_dtype DT, int GROUP, int CIF>
hipError_t launch_segreduce_g(dim3 grid, float* out, int64_t H, const void* src, const int32_t* perm,
                              const TileRec* tiles, float* partials, int tc_log2, int64_t slices, int32_t* status,
                              uint64_t* fp_part, hipStream_t s) {
#define DR_SEGREDUCE_CASE(TC)                                                                                  \
    case TC:                                                                                                   \
        hipLaunchKernelGGL((segreduce_kernel<DT, GROUP, TC, CIF>), grid, dim3(kReduceThreads), 0, s, out, H,    \
                           src, perm, tiles, partials, slices, status, fp_part);                               \
        break;
    switch (tc_log2) {
        DR_SEGREDUCE_CASE(3)
        DR_SEGREDUCE_CASE(4)
        DR_SEGREDUCE_CASE(5)
        DR_SEGREDUCE_CASE(6)
        DR_SEGREDUCE_CASE(7)
        default:
            return hipErrorInvalidValue;
    }
#undef DR_SEGREDUCE_CASE
    return hipGetLastError();
}

// Columns per lane of the formed-contribution reduce: the fewest (at least 2)
// that cover the row with one wavefront, capped at 16 bytes per lane.
template <dr_dtype DT, int E>
hipError_t launch_gen_e(dim3 grid, float* out, int64_t H, const void* src, const int32_t* perm,
                        const TileRec* tiles, float* partials, int tc_log2, const int32_t* status, const float* scale,
                        bool scale_sorted, uint32_t rps, hipStream_t s) {
    const int64_t slices = (H + 64 * E - 1) / (64 * E);
    // p / rps as a multiply and shift (gen_row_of); rps >= 1
    uint32_t sh = 0;
    while (((uint64_t)1 << sh) < rps) ++sh;
    const uint32_t m = (uint32_t)((((uint64_t)1 << (31 + sh)) + rps - 1) / rps);
#define DR_GEN_CASE(TC)                                                                                         \
    case TC:                                                                                                    \
        if (scale_sorted)                                                                                       \
            hipLaunchKernelGGL((segreduce_gen_kernel<DT, E, TC, true>), grid, dim3(kReduceThreads), 0, s, out,   \
                               H, static_cast<const char*>(src), perm, tiles, partials, slices, status, scale,  \
                               m, sh);                                                                          \
        else                                                                                                    \
            hipLaunchKernelGGL((segreduce_gen_kernel<DT, E, TC, false>), grid, dim3(kReduceThreads), 0, s, out,  \
                               H, static_cast<const char*>(src), perm, tiles, partials, slices, status, scale,  \
                               m, sh);                                                                          \
        break;
    switch (tc_log2) {
        DR_GEN_CASE(3)
        DR_GEN_CASE(4)
        DR_GEN_CASE(5)
        DR_GEN_CASE(6)
        DR_GEN_CASE(7)
        default:
            return hipErrorInvalidValue;
    }
#undef DR_GEN_CASE
    return hipGetLastError();
}

template <bool SORTED, bool POW2>
hipError_t launch_gen16(dim3 grid, float* out, int64_t H, const void* src, uint32_t src_bytes, const int32_t* perm,
                        uint32_t n, const TileRec* tiles, float* partials, int tc_log2, const int32_t* status,
                        const float* scale, uint32_t m, uint32_t sh, hipStream_t s) {
    const int64_t slices = (H + 127) / 128;
#define DR_GEN16_CASE(TC)                                                                                       \
    case TC:                                                                                                    \
        hipLaunchKernelGGL((segreduce_gen16_kernel<TC, SORTED, POW2>), grid, dim3(kReduceThreads), 0, s, out,   \
                           H, static_cast<const char*>(src), src_bytes, perm, n, tiles, partials, slices,       \
                           status, scale, m, sh);                                                               \
        break;
    switch (tc_log2) {
        DR_GEN16_CASE(3)
        DR_GEN16_CASE(4)
        DR_GEN16_CASE(5)
        DR_GEN16_CASE(6)
        DR_GEN16_CASE(7)
        default:
            return hipErrorInvalidValue;
    }
#undef DR_GEN16_CASE
    return hipGetLastError();
}

hipError_t launch_segreduce_gen(dim3 grid, float* out, int64_t H, const void* src, int64_t src_rows, int64_t n,
                                dr_dtype dt, const int32_t* perm, const TileRec* tiles, float* partials, int tc_log2,
                                const int32_t* status, const float* scale, bool scale_sorted, uint32_t rps,
                                hipStream_t s) {
    // bf16 source rows of fewer than 2^31 bytes in all take the LDS form (32-bit
    // buffer offsets, formed by 24-bit multiplies: fewer than 2^24 rows of fewer
    // than 2^24 bytes)
    const int64_t src_bytes = src_rows * H * 2;
    if (dt == DR_BF16 && src_bytes < ((int64_t)1 << 31) && n < ((int64_t)1 << 29) && src_rows < ((int64_t)1 << 24) &&
        H * 2 < ((int64_t)1 << 24)) {
        uint32_t sh = 0;
        while (((uint64_t)1 << sh) < rps) ++sh;
        const uint32_t m = (uint32_t)((((uint64_t)1 << (31 + sh)) + rps - 1) / rps);
        const bool pow2 = (rps & (rps - 1)) == 0;
        const uint32_t sb = (uint32_t)src_bytes, nn = (uint32_t)n;
        if (scale_sorted)
            return pow2 ? launch_gen16<true, true>(grid, out, H, src, sb, perm, nn, tiles, partials, tc_log2, status,
                                                   scale, m, sh, s)
                        : launch_gen16<true, false>(grid, out, H, src, sb, perm, nn, tiles, partials, tc_log2, status,
                                                    scale, m, sh, s);
        return pow2 ? launch_gen16<false, true>(grid, out, H, src, sb, perm, nn, tiles, partials, tc_log2, status,
                                                scale, m, sh, s)
                    : launch_gen16<false, false>(grid, out, H, src, sb, perm, nn, tiles, partials, tc_log2, status,
                                                 scale, m, sh, s);
    }
    if (dt == DR_BF16) {
        if (H <= 128) return launch_gen_e<DR_BF16, 2>(grid, out, H, src, perm, tiles, partials, tc_log2, status, scale,
                                                      scale_sorted, rps, s);
        if (H <= 256) return launch_gen_e<DR_BF16, 4>(grid, out, H, src, perm, tiles, partials, tc_log2, status, scale,
                                                      scale_sorted, rps, s);
        return launch_gen_e<DR_BF16, 8>(grid, out, H, src, perm, tiles, partials, tc_log2, status, scale,
                                        scale_sorted, rps, s);
    }
    if (H <= 128) return launch_gen_e<DR_F32, 2>(grid, out, H, src, perm, tiles, partials, tc_log2, status, scale,
                                                 scale_sorted, rps, s);
    return launch_gen_e<DR_F32, 4>(grid, out, H, src, perm, tiles, partials, tc_log2, status, scale, scale_sorted,
                                   rps, s);
}

}  // namespace

unsigned persistent_grid() {
    const Launch lc = launch_config();
    if (lc.grid_blocks > 0) return (unsigned)lc.grid_blocks;
    return (unsigned)(device_cu_count() * 16);
}

int64_t plan_blocks(int32_t num_dests) { return ((int64_t)num_dests + kPlanThreads - 1) / kPlanThreads; }

hipError_t launch_plan_count(const int32_t* seg_offsets, int32_t num_dests, int64_t n, int tc_log2,
                             int32_t* block_sums, int32_t* status, hipStream_t s) {
    hipLaunchKernelGGL(plan_count_kernel, dim3((unsigned)plan_blocks(num_dests)), dim3(kPlanThreads), 0, s,
                       seg_offsets, num_dests, n, tc_log2, block_sums, status);
    return hipGetLastError();
}

hipError_t launch_plan_count_search(const int32_t* sorted_dest, int64_t n, int32_t num_dests, int tc_log2,
                                    int32_t* seg_offsets, int32_t* block_sums, int32_t* status, hipStream_t s) {
    hipLaunchKernelGGL(plan_count_search_kernel, dim3((unsigned)plan_blocks(num_dests)), dim3(kPlanThreads), 0, s,
                       sorted_dest, n, num_dests, tc_log2, seg_offsets, block_sums, status);
    return hipGetLastError();
}

hipError_t launch_plan_write(const int32_t* seg_offsets, int32_t num_dests, int tc_log2, const int32_t* block_sums,
                             TileRec* tiles, MultiRec* multis, int32_t* status, hipStream_t s) {
    hipLaunchKernelGGL(plan_write_kernel, dim3((unsigned)plan_blocks(num_dests)), dim3(kPlanThreads), 0, s,
                       seg_offsets, num_dests, tc_log2, block_sums, tiles, multis, status);
    return hipGetLastError();
}

hipError_t launch_plan_validate(const int32_t* perm, const int32_t* seg, const int32_t* index, int64_t n,
                                int32_t num_dests, int32_t* status, hipStream_t s) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(plan_validate_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, perm, seg, index, n,
                       num_dests, status);
    return hipGetLastError();
}

hipError_t launch_segreduce(float* out, int64_t hidden, const void* src, dr_dtype dt, int64_t n, const int32_t* perm,
                            const TileRec* tiles, float* partials, int tc_log2, int cif, const float* scale,
                            bool scale_sorted, int32_t rows_per_src, int32_t* status, uint64_t* fp_part,
                            hipStream_t s) {
    const int64_t lanes = dt == DR_BF16 ? hidden / 8 : hidden / 4;  // lanes needed per row
    const int g = group_for(lanes);
    const int64_t slices = (lanes + g - 1) / g;
    const dim3 grid(persistent_grid());
    const uint32_t rps = (uint32_t)rows_per_src;
    if (scale) {
        if (fp_part) return hipErrorInvalidValue;  // formed contributions keep no fingerprint
        return launch_segreduce_gen(grid, out, hidden, src, (n + rows_per_src - 1) / rows_per_src, n, dt, perm,
                                    tiles, partials, tc_log2, status, scale, scale_sorted, rps, s);
    }
#define DR_SR(DT, G)                                                                                           \
    return cif == 1 ? launch_segreduce_g<DT, G, 1>(grid, out, hidden, src, perm, tiles, partials, tc_log2,     \
                                                   slices, status, fp_part, s)                                 \
                    : launch_segreduce_g<DT, G, 2>(grid, out, hidden, src, perm, tiles, partials, tc_log2,     \
                                                   slices, status, fp_part, s)
    if (dt == DR_BF16) {
        if (g == 16) { DR_SR(DR_BF16, 16); }
        if (g == 32) { DR_SR(DR_BF16, 32); }
        DR_SR(DR_BF16, 64);
    }
    if (g == 16) { DR_SR(DR_F32, 16); }
    if (g == 32) { DR_SR(DR_F32, 32); }
    DR_SR(DR_F32, 64);
#undef DR_SR
}

hipError_t launch_tilecombine(float* out, int64_t hidden, const float* partials, const MultiRec* multis, int64_t n,
                              int tc_log2, int32_t* status, uint64_t* fp_part, hipStream_t s) {
    const int64_t slices = (hidden + 127) / 128;
    const dim3 grid(persistent_grid());
    // the most tiles one destination can have, and the counter depth it needs
    const int64_t max_tiles = n / ((int64_t)8 << tc_log2) + 1;
    int depth = 1;
    while (depth < 62 && ((int64_t)1 << depth) <= max_tiles) ++depth;
    if (depth > 32) return hipErrorInvalidValue;
#define DR_TC(D) \
    hipLaunchKernelGGL((tilecombine_kernel<D>), grid, dim3(kReduceThreads), 0, s, out, hidden, partials, multis, slices, \
                       status, fp_part)
    if (depth <= 8) DR_TC(8);
    else if (depth <= 16) DR_TC(16);
    else DR_TC(32);
#undef DR_TC
    return hipGetLastError();
}

}  // namespace dr
