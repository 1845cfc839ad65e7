// Stable LSD radix sort of contributions by (destination, source id), and the
// CSR segment offsets of the sorted order.
//
// The order it produces is the one the DeepSeek-V4 MoE backward uses (ch. 9,
// section 3.2: sort the tokens that land on a rank by (expert_id,
// original_token_id) and merge in that order).  Stability comes from ranking
// keys inside a workgroup in index order.  Integer atomics only count
// histogram entries, whose totals do not depend on the order of the
// increments; no atomic ever claims an output slot.
//
// Pass structure (per digit of up to 9 bits):
//   radix_hist:    digit counts of each tile of keys (LDS, wave-aggregated).
//                  The first pass also checks every index and leaves one
//                  error flag per tile.
//   radix_scan:    one workgroup per digit scans that digit's counts over the
//                  tiles; totals per digit.  On the first pass one more
//                  workgroup folds the tile flags into the call's status word
//                  (set or cleared), so no separate reset launch is needed.
//   radix_scatter: recomputes each key's stable rank inside its tile, stages
//                  the tile in LDS in digit order, then writes each digit's run
//                  to consecutive output positions (coalesced stores).  When
//                  the pass's digit is the whole destination (one dest pass),
//                  workgroup 0 also writes the segment offsets, which are the
//                  digit prefix sums it has already formed.
#include "internal.h"

namespace dr {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxBins = 1 << kMaxDigitBits;
constexpr int64_t kXcds = 8;  // XCDs of an MI355X, each with its own L2

__device__ __forceinline__ int digit_of(int32_t key, int shift, int bits) {
    return (int)(((uint32_t)key >> shift) & ((1u << bits) - 1u));
}

__device__ __forceinline__ int32_t wave_inclusive_scan(int32_t v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        int32_t t = __shfl_up(v, off, 64);
        if (lane >= off) v += t;
    }
    return v;
}

// Exclusive scan over the workgroup (kThreads threads); total gets the sum.
__device__ int32_t block_exclusive_scan(int32_t v, int32_t& total, int32_t* wave_tot) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int32_t incl = wave_inclusive_scan(v);
    if (lane == 63) wave_tot[w] = incl;
    __syncthreads();
    int32_t before = 0, all = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
        const int32_t s = wave_tot[i];
        before += (i < w) ? s : 0;
        all += s;
    }
    __syncthreads();
    total = all;
    return before + incl - v;
}

// Exclusive scan of bins (<= 2 * kThreads) values held in LDS, in place.
__device__ void scan_bins_in_place(int32_t* a, int bins, int32_t* wave_tot) {
    // thread t owns bins 2t and 2t+1
    const int t = threadIdx.x;
    const int32_t x0 = 2 * t < bins ? a[2 * t] : 0;
    const int32_t x1 = 2 * t + 1 < bins ? a[2 * t + 1] : 0;
    int32_t total;
    const int32_t ex = block_exclusive_scan(x0 + x1, total, wave_tot);
    if (2 * t < bins) a[2 * t] = ex;
    if (2 * t + 1 < bins) a[2 * t + 1] = ex + x0;
    __syncthreads();
}

__global__ void fill_status_kernel(int32_t* status) {
    if (threadIdx.x < kStatusBytes / sizeof(int32_t)) status[threadIdx.x] = 0;
}

// Digit histogram of one tile of keys per workgroup.  Every thread first
// loads its ITEMS keys (all loads in flight together), then counts them in
// LDS; a wavefront whose keys all share one digit adds once.  With kValidate,
// also checks every dest (and src_id) against its range: the first pass.
// HT threads per workgroup: 1024 for tiles of at least 2^10 keys, so that a
// CU holds more wavefronts to hide the key loads.
template <bool kValidate, int HT, int ITEMS>
__global__ __launch_bounds__(HT) void radix_hist_kernel(SortPass p, int64_t n, int tile_log2, int32_t* hist,
                                                        int64_t nblocks, const int32_t* __restrict__ dest,
                                                        int32_t num_dests, const int32_t* __restrict__ src_id,
                                                        int32_t src_bound, int32_t* status_or_flags) {
    __shared__ int32_t cnt[kMaxBins];
    __shared__ int32_t bad;
    // later passes: status word (same value for every thread); first pass: tile flags
    if (!kValidate && status_or_flags[kWordStatus] != 0) return;
    const int bins = 1 << p.bits;
    for (int d = threadIdx.x; d < bins; d += HT) cnt[d] = 0;
    if (threadIdx.x == 0) bad = 0;
    const int64_t base = (int64_t)blockIdx.x << tile_log2;
    const int64_t end = min(n, base + ((int64_t)1 << tile_log2));
    int32_t key[ITEMS];
    int my_bad = 0;
#pragma unroll
    for (int r = 0; r < ITEMS; ++r) {
        const int64_t i = base + r * HT + threadIdx.x;
        key[r] = i < end ? p.digit_src[i] : 0;
        if (kValidate && i < end) {
            const int32_t dd = dest[i];
            my_bad |= (dd < 0 || dd >= num_dests);
            if (src_id) {
                const int32_t ss = src_id[i];
                my_bad |= (ss < 0 || ss >= src_bound);
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < ITEMS; ++r) {
        const int64_t i = base + r * HT + threadIdx.x;
        const bool valid = i < end;
        const int dg = digit_of(key[r], p.shift, p.bits);
        const uint64_t vmask = __ballot(valid);
        const int first = __builtin_amdgcn_readfirstlane(dg);
        if (vmask != 0 && __ballot(valid && dg == first) == vmask) {
            if ((threadIdx.x & 63) == __builtin_ctzll(vmask)) atomicAdd(&cnt[first], (int32_t)__popcll(vmask));
        } else if (valid) {
            atomicAdd(&cnt[dg], 1);
        }
    }
    if (my_bad) bad = 1;
    __syncthreads();
    for (int d = threadIdx.x; d < bins; d += HT) hist[(int64_t)d * nblocks + blockIdx.x] = cnt[d];
    if (kValidate && threadIdx.x == 0) status_or_flags[blockIdx.x] = bad;
}

// One workgroup per digit: exclusive scan of that digit's counts over the
// tiles (in place), and the digit's total.  With tile_flags (first pass), the
// last workgroup writes the status word from the flags instead; the digit
// workgroups then scan regardless (the counts stay consistent for any key).
__global__ __launch_bounds__(kThreads) void radix_scan_kernel(int32_t* hist, int64_t nblocks, int32_t* totals,
                                                              int32_t* status, const int32_t* tile_flags) {
    __shared__ int32_t wave_tot[kWaves];
    if (tile_flags) {
        if (blockIdx.x == gridDim.x - 1) {
            int32_t any = 0;
            for (int64_t b = threadIdx.x; b < nblocks; b += kThreads) any |= tile_flags[b];
            any = __syncthreads_or(any);
            if (threadIdx.x == 0) status[kWordStatus] = any ? kStatusIndex : 0;
            return;
        }
    } else if (status[kWordStatus] != 0) {
        return;
    }
    int32_t* h = hist + (int64_t)blockIdx.x * nblocks;
    int32_t carry = 0;
    for (int64_t b0 = 0; b0 < nblocks; b0 += kThreads) {
        const int64_t b = b0 + threadIdx.x;
        const int32_t v = b < nblocks ? h[b] : 0;
        int32_t tot;
        const int32_t ex = block_exclusive_scan(v, tot, wave_tot);
        if (b < nblocks) h[b] = carry + ex;
        carry += tot;
    }
    if (threadIdx.x == 0) totals[blockIdx.x] = carry;
}

// Stable scatter of one tile.  Wavefront w owns the contiguous slice
// [64*ITEMS*w, 64*ITEMS*(w+1)) of the tile and visits it in ITEMS rounds of 64
// consecutive keys.  A key's rank among equal digits of its wavefront is the
// wavefront's count of that digit in earlier rounds (a per-wavefront LDS
// counter, no barrier) plus the lower lanes of its round with the same digit
// (a per-wavefront LDS table of lane masks by digit).  One barrier later, the
// tile rank adds the counts of earlier wavefronts; equal digits therefore keep
// input order.  The tile is staged in
// LDS in (digit, rank) order and each digit's run is written to consecutive
// global positions.
template <int ITEMS, int BINS, bool STAGE_SRC, bool PAY>
__global__ __launch_bounds__(kThreads) void radix_scatter_kernel(SortPass p, int64_t n, int tile_log2,
                                                                 const int32_t* __restrict__ hist, int64_t nblocks,
                                                                 const int32_t* __restrict__ totals,
                                                                 const int32_t* status) {
    __shared__ int32_t gbase[BINS];          // global position of this tile's first key of digit d
    __shared__ int32_t lbase[BINS];          // position of digit d's run inside the staged tile
    __shared__ int32_t wcount[kWaves][BINS];  // per-wavefront digit counts, then prefixes
    __shared__ int32_t wave_tot[kWaves];
    // The staged tile, and before it (ranking only) each wavefront's table of
    // lane masks by digit.
    constexpr int kStageBytes = (2 + (STAGE_SRC ? 1 : 0) + (PAY ? 1 : 0)) * ITEMS * kThreads * 4;
    constexpr int kTableBytes = kWaves * BINS * 8;
    __shared__ __align__(16) unsigned char shared_un[kStageBytes > kTableBytes ? kStageBytes : kTableBytes];
    int32_t* st_dest = reinterpret_cast<int32_t*>(shared_un);
    int32_t* st_val = st_dest + ITEMS * kThreads;
    int32_t* st_src = st_val + ITEMS * kThreads;
    float* st_pay = reinterpret_cast<float*>(st_val + (STAGE_SRC ? 2 : 1) * ITEMS * kThreads);
    if (status[kWordStatus] != 0) return;
    // Workgroups are spread over the XCDs round-robin (workgroup b on XCD
    // b % kXcds); each XCD takes a contiguous range of tiles, so the digit runs
    // that neighbouring tiles write next to each other mostly meet in one L2
    // and leave it as whole lines.  The grid is kXcds * per workgroups; the few
    // past the last tile do nothing.
    const int64_t per = (nblocks + kXcds - 1) / kXcds;
    const int64_t tile = (int64_t)(blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
    if (tile >= nblocks) return;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    unsigned long long* peer_tbl = reinterpret_cast<unsigned long long*>(shared_un) + w * BINS;
    const int bins = 1 << p.bits;
    const bool key_is_dest = p.digit_src == p.dest_in;
    const int64_t base = tile << tile_log2;
    const int64_t end = min(n, base + ((int64_t)1 << tile_log2));
    const int32_t count = (int32_t)(end - base);
    const int64_t wbase = base + (int64_t)w * 64 * ITEMS;  // this wavefront's slice

    // this thread's keys, values and carried ids, all loads in flight together
    int32_t key[ITEMS], other[ITEMS], val[ITEMS];
    float pay[PAY ? ITEMS : 1];
#pragma unroll
    for (int r = 0; r < ITEMS; ++r) {
        const int64_t i = wbase + r * 64 + lane;
        key[r] = other[r] = 0;
        val[r] = (int32_t)i;
        if (PAY) pay[r] = 0.f;
        if (i < end) {
            key[r] = p.digit_src[i];
            other[r] = key_is_dest ? (STAGE_SRC ? p.src_in[i] : 0) : p.dest_in[i];
            if (p.val_in) val[r] = p.val_in[i];
            if (PAY) pay[r] = p.pay_in[i];
        }
    }
    for (int d = tid; d < bins; d += kThreads) {
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) wcount[ww][d] = 0;
        gbase[d] = totals[d];
    }
    for (int d = lane; d < bins; d += 64) peer_tbl[d] = 0ull;  // this wavefront's table
    __syncthreads();

    // ranks inside the wavefront, in input order.  The lanes holding a digit
    // are found by each lane OR-ing its bit into the digit's entry of the
    // wavefront's table, reading the entry back and clearing it (a
    // wavefront's LDS operations complete in order, and OR does not depend on
    // the order of the lanes); this replaces one ballot per digit bit.
    const unsigned long long my_bit = 1ull << lane;
    int32_t rank[ITEMS];
#pragma unroll
    for (int r = 0; r < ITEMS; ++r) {
        const bool valid = wbase + r * 64 + lane < end;
        const int dg = digit_of(key[r], p.shift, p.bits);
        uint64_t peers = 0;
        if (valid) {
            atomicOr(&peer_tbl[dg], my_bit);
            peers = peer_tbl[dg];
            peer_tbl[dg] = 0ull;
        }
        const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(peers >> 32),
                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)peers, 0u));
        // every lane of the digit reads the count (one instruction) before the
        // lowest of them advances it
        int32_t prev = 0;
        if (valid) prev = wcount[w][dg];
        if (valid && below == 0) wcount[w][dg] = prev + (int32_t)__popcll(peers);
        rank[r] = prev + below;
    }
    __syncthreads();
    // per digit: tile count, offsets of the wavefronts, and the global base
    for (int d = tid; d < bins; d += kThreads) {
        int32_t acc = 0;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) {
            const int32_t c = wcount[ww][d];
            wcount[ww][d] = acc;
            acc += c;
        }
        lbase[d] = acc;  // the tile's count of digit d, scanned below
    }
    __syncthreads();
    scan_bins_in_place(gbase, bins, wave_tot);
    scan_bins_in_place(lbase, bins, wave_tot);
    // gbase[d] now counts all keys of digits below d.  From here on gbase[d]
    // is the global position of staged position 0 of digit d's run, and
    // wcount[w][d] the staged position of wavefront w's first key of digit d.
    int32_t* seg = tile == 0 ? p.seg_out : nullptr;
    for (int d = tid; d < bins; d += kThreads) {
        if (seg && d <= p.num_dests) seg[d] = gbase[d];
        const int32_t lb = lbase[d];
        gbase[d] += hist[(int64_t)d * nblocks + tile] - lb;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) wcount[ww][d] += lb;
    }
    if (seg && tid == 0 && p.num_dests == bins) seg[bins] = (int32_t)n;
    __syncthreads();
#pragma unroll
    for (int r = 0; r < ITEMS; ++r) {
        if (wbase + r * 64 + lane < end) {
            const int dg = digit_of(key[r], p.shift, p.bits);
            const int32_t lp = wcount[w][dg] + rank[r];
            st_val[lp] = val[r];
            st_dest[lp] = key_is_dest ? key[r] : other[r];
            if (STAGE_SRC) st_src[lp] = key_is_dest ? other[r] : key[r];
            if (PAY) st_pay[lp] = pay[r];
        }
    }
    __syncthreads();
    // write-out in staged order: a digit's run goes to consecutive positions
    for (int32_t j = tid; j < count; j += kThreads) {
        const int32_t dk = st_dest[j];
        const int32_t sk = STAGE_SRC ? st_src[j] : 0;
        const int dg = digit_of(key_is_dest ? dk : sk, p.shift, p.bits);
        const int32_t pos = gbase[dg] + j;
        const int32_t v = st_val[j];
        // consistent histograms keep pos and v inside [0, n); the guard keeps
        // a corrupted workspace from writing outside the outputs
        if ((uint64_t)(uint32_t)pos >= (uint64_t)n || (uint64_t)(uint32_t)v >= (uint64_t)n) continue;
        p.val_out[pos] = v;
        if (p.dest_out) p.dest_out[pos] = dk;
        if (STAGE_SRC && p.src_out) p.src_out[pos] = sk;
        if (PAY) p.pay_out[pos] = st_pay[j];
        if (p.inv_out) p.inv_out[v] = pos;
    }
}

// seg_offsets[d] = first sorted position whose dest is >= d (lower bound),
// for d = 0 .. num_dests; sorted_dest is non-decreasing.
__global__ void seg_offsets_kernel(const int32_t* __restrict__ sorted_dest, int64_t n, int32_t num_dests,
                                   int32_t* __restrict__ seg, const int32_t* status) {
    if (status[kWordStatus] != 0) return;
    const int64_t d = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (d > num_dests) return;
    int64_t lo = 0, hi = n;
    while (lo < hi) {
        const int64_t mid = (lo + hi) >> 1;
        if (sorted_dest[mid] < d) lo = mid + 1;
        else hi = mid;
    }
    seg[d] = (int32_t)lo;
}

}  // namespace

hipError_t launch_fill_status(int32_t* status_block, hipStream_t s) {
    hipLaunchKernelGGL(fill_status_kernel, dim3(1), dim3(64), 0, s, status_block);
    return hipGetLastError();
}

static int64_t tiles_for(int64_t n, int tile_log2) { return (n + ((int64_t)1 << tile_log2) - 1) >> tile_log2; }

#define DR_BY_ITEMS(tile_log2, MACRO) \
    switch (tile_log2) {                 \
        case 8: MACRO(1); break;         \
        case 9: MACRO(2); break;         \
        case 10: MACRO(4); break;        \
        case 11: MACRO(8); break;        \
        case 12: MACRO(16); break;       \
        default: MACRO(32); break;       \
    }

#define DR_HIST_BY_TILE(tile_log2, MACRO) \
    switch (tile_log2) {                       \
        case 8: MACRO(256, 1); break;          \
        case 9: MACRO(256, 2); break;          \
        case 10: MACRO(1024, 1); break;        \
        case 11: MACRO(1024, 2); break;        \
        case 12: MACRO(1024, 4); break;        \
        default: MACRO(1024, 8); break;        \
    }

hipError_t launch_radix_validate_hist(const int32_t* dest, int32_t num_dests, const int32_t* src_id,
                                      int32_t src_bound, const SortPass& p, int64_t n, int tile_log2,
                                      int32_t* hist, int32_t* tile_flags, hipStream_t s) {
    const int64_t nb = tiles_for(n, tile_log2);
    if (nb == 0) return hipSuccess;
#define DR_H(HTH, IT)                                                                                         \
    hipLaunchKernelGGL((radix_hist_kernel<true, HTH, IT>), dim3((unsigned)nb), dim3(HTH), 0, s, p, n, tile_log2, \
                       hist, nb, dest, num_dests, src_id, src_bound, tile_flags)
    DR_HIST_BY_TILE(tile_log2, DR_H)
#undef DR_H
    return hipGetLastError();
}

hipError_t launch_radix_hist(const SortPass& p, int64_t n, int tile_log2, int32_t* hist, const int32_t* status,
                             hipStream_t s) {
    const int64_t nb = tiles_for(n, tile_log2);
    if (nb == 0) return hipSuccess;
#define DR_H(HTH, IT)                                                                                          \
    hipLaunchKernelGGL((radix_hist_kernel<false, HTH, IT>), dim3((unsigned)nb), dim3(HTH), 0, s, p, n, tile_log2, \
                       hist, nb, nullptr, 0, nullptr, 0, const_cast<int32_t*>(status))
    DR_HIST_BY_TILE(tile_log2, DR_H)
#undef DR_H
    return hipGetLastError();
}

hipError_t launch_radix_scan(int32_t* hist, int64_t nblocks, int bins, int32_t* totals, int32_t* status,
                             const int32_t* tile_flags, hipStream_t s) {
    if (nblocks == 0) return hipSuccess;
    hipLaunchKernelGGL(radix_scan_kernel, dim3(bins + (tile_flags ? 1 : 0)), dim3(kThreads), 0, s, hist, nblocks,
                       totals, status, tile_flags);
    return hipGetLastError();
}

template <int ITEMS>
static void launch_scatter_items(const SortPass& p, int64_t n, int tile_log2, const int32_t* hist,
                                 const int32_t* totals, const int32_t* status, int64_t nb, hipStream_t s) {
    const bool stage_src = p.src_out != nullptr || p.digit_src != p.dest_in;
    const bool pay = p.pay_out != nullptr;  // the host never asks for a payload together with source ids
    const dim3 grid((unsigned)(kXcds * ((nb + kXcds - 1) / kXcds))), block(kThreads);
#define DR_SC(BINS, SRC, PY)                                                                                      \
    hipLaunchKernelGGL((radix_scatter_kernel<ITEMS, BINS, SRC, PY>), grid, block, 0, s, p, n, tile_log2, hist, nb, \
                       totals, status)
    if (p.bits <= 8) {
        if (stage_src) DR_SC(256, true, false);
        else if (pay) DR_SC(256, false, true);
        else DR_SC(256, false, false);
    } else {
        if (stage_src) DR_SC(kMaxBins, true, false);
        else if (pay) DR_SC(kMaxBins, false, true);
        else DR_SC(kMaxBins, false, false);
    }
#undef DR_SC
}

hipError_t launch_radix_scatter(const SortPass& p, int64_t n, int tile_log2, const int32_t* hist,
                                const int32_t* totals, const int32_t* status, hipStream_t s) {
    const int64_t nb = tiles_for(n, tile_log2);
    if (nb == 0) return hipSuccess;
    if ((p.pay_out != nullptr) != (p.pay_in != nullptr) || (p.pay_out && (p.src_out || p.digit_src != p.dest_in)))
        return hipErrorInvalidValue;
    // the staged tile (dest, value and a source id or a payload of 2^13 keys: 96 KB) plus
    // counters stays within a gfx950 workgroup's 160 KB of LDS
    static_assert(kMaxSortTileLog2 <= 13, "staged tile must fit in LDS");
#define DR_S(IT) launch_scatter_items<IT>(p, n, tile_log2, hist, totals, status, nb, s)
    DR_BY_ITEMS(tile_log2, DR_S)
#undef DR_S
    return hipGetLastError();
}

hipError_t launch_seg_offsets(const int32_t* sorted_dest, int64_t n, int32_t num_dests, int32_t* seg_offsets,
                              const int32_t* status, hipStream_t s) {
    const int64_t count = (int64_t)num_dests + 1;
    const unsigned blocks = (unsigned)((count + kThreads - 1) / kThreads);
    hipLaunchKernelGGL(seg_offsets_kernel, dim3(blocks), dim3(kThreads), 0, s, sorted_dest, n, num_dests,
                       seg_offsets, status);
    return hipGetLastError();
}

}  // namespace dr
