// C-ABI layer of libdetreduce: argument validation (fail closed, nothing is
// launched on a bad argument), workspace layout, and the order of kernel
// launches for each entry point.  See include/detreduce.h for the contract.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "internal.h"

namespace {

thread_local std::string g_err;
thread_local dr_launch_params g_params = {0, 0, 0, 0, 0};
thread_local hipEvent_t g_reduce_begin = nullptr, g_reduce_end = nullptr;  // dr_set_phase_events

dr_status fail(dr_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return s;
}

dr_status ok() {
    g_err.clear();
    return DR_OK;
}

dr_status hip_fail(hipError_t e, const char* what) {
    return fail(DR_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define DR_TRY_HIP(expr, what)                        \
    do {                                              \
        hipError_t e_ = (expr);                       \
        if (e_ != hipSuccess) return hip_fail(e_, what); \
    } while (0)

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

// Carves a workspace into aligned slices; with base == nullptr it only sizes.
struct Carver {
    char* base;
    size_t off = 0;
    explicit Carver(void* b) : base(static_cast<char*>(b)) {}
    template <typename T>
    T* take(int64_t count) {
        T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
        off += align_up((size_t)(count > 0 ? count : 0) * sizeof(T));
        return p;
    }
};

int bitwidth(uint32_t x) {
    int b = 0;
    while (x) {
        ++b;
        x >>= 1;
    }
    return b;
}

struct DigitPass {
    bool from_src;
    int shift;
    int bits;
};

// LSD passes: source-id digits first (least significant), then destination digits.
std::vector<DigitPass> sort_passes(int32_t num_dests, bool has_src, int32_t src_bound) {
    std::vector<DigitPass> passes;
    auto add = [&](bool from_src, int total_bits) {
        if (total_bits <= 0) return;
        const int np = (total_bits + dr::kMaxDigitBits - 1) / dr::kMaxDigitBits;
        const int width = (total_bits + np - 1) / np;
        for (int shift = 0; shift < total_bits; shift += width)
            passes.push_back({from_src, shift, std::min(width, total_bits - shift)});
    };
    if (has_src) add(true, bitwidth((uint32_t)(src_bound - 1)));
    add(false, bitwidth((uint32_t)(num_dests - 1)));
    if (passes.empty()) passes.push_back({false, 0, 1});  // one destination: a single stable pass
    return passes;
}

struct SortBuffers {
    int32_t* hist;
    int32_t* tile_flags;  // first pass: index-error flag per tile
    int32_t* totals;
    int32_t *dest_a, *dest_b, *val_a, *val_b, *src_a, *src_b;
    float *pay_a, *pay_b;  // a payload moved with the keys (optional)
    int64_t nblocks;
};

SortBuffers carve_sort(Carver& c, int64_t n, bool has_src, int tile_log2, bool has_pay = false) {
    SortBuffers b{};
    b.nblocks = (n + ((int64_t)1 << tile_log2) - 1) >> tile_log2;
    b.hist = c.take<int32_t>((int64_t)(1 << dr::kMaxDigitBits) * b.nblocks);
    b.tile_flags = c.take<int32_t>(b.nblocks);
    b.totals = c.take<int32_t>(1 << dr::kMaxDigitBits);
    b.dest_a = c.take<int32_t>(n);
    b.dest_b = c.take<int32_t>(n);
    b.val_a = c.take<int32_t>(n);
    b.val_b = c.take<int32_t>(n);
    b.src_a = has_src ? c.take<int32_t>(n) : nullptr;
    b.src_b = has_src ? c.take<int32_t>(n) : nullptr;
    b.pay_a = has_pay ? c.take<float>(n) : nullptr;
    b.pay_b = has_pay ? c.take<float>(n) : nullptr;
    return b;
}

// Launches the stable sort.  It writes the status word itself (the first
// pass's scan sets or clears the index-error bit), so no reset launch is
// needed before it.
// With seg_deferred, segment offsets that would need a separate search are
// left to the caller: *seg_deferred is then true and *sorted_dest_out the
// sorted destinations (not read when n == 0); otherwise seg_offsets is
// written here.  With pay (no source ids then, and buffers carved for it),
// pay[i] moves with key i and *pay_sorted_out receives the sorted payload.
dr_status run_sort(const int32_t* dest, const int32_t* src_id, int32_t src_bound, int64_t n, int32_t num_dests,
                   int32_t* perm, int32_t* seg_offsets, int32_t* inv_perm, int32_t* status, const SortBuffers& b,
                   int tile_log2, hipStream_t s, bool* seg_deferred = nullptr,
                   const int32_t** sorted_dest_out = nullptr, const float* pay = nullptr,
                   const float** pay_sorted_out = nullptr) {
    const bool has_src = src_id != nullptr;
    const std::vector<DigitPass> passes = sort_passes(num_dests, has_src, src_bound);
    int src_passes = 0;
    for (const DigitPass& p : passes) src_passes += p.from_src;
    // with no keys no pass runs: the status is cleared here instead
    if (n == 0) DR_TRY_HIP(dr::launch_fill_status(status, s), "status reset launch");
    // a single destination pass sees whole destinations: its scatter writes seg_offsets
    const bool seg_in_scatter = n > 0 && (int)passes.size() - src_passes == 1;
    const int32_t* cur_dest = dest;
    const int32_t* cur_src = src_id;
    const int32_t* cur_val = nullptr;
    const float* cur_pay = pay;
    for (size_t i = 0; i < passes.size(); ++i) {
        const bool last = i + 1 == passes.size();
        const bool odd = i & 1;
        const bool carry_src = has_src && (int)i + 1 < src_passes;
        dr::SortPass sp{};
        sp.digit_src = passes[i].from_src ? cur_src : cur_dest;
        sp.shift = passes[i].shift;
        sp.bits = passes[i].bits;
        sp.dest_in = cur_dest;
        // the last pass's sorted keys are only needed by the segment-offset search
        sp.dest_out = last && seg_in_scatter ? nullptr : (odd ? b.dest_b : b.dest_a);
        sp.src_in = (carry_src || passes[i].from_src) ? cur_src : nullptr;
        sp.src_out = carry_src ? (odd ? b.src_b : b.src_a) : nullptr;
        sp.val_in = cur_val;
        sp.val_out = last ? perm : (odd ? b.val_b : b.val_a);
        sp.inv_out = last ? inv_perm : nullptr;
        sp.seg_out = last && seg_in_scatter ? seg_offsets : nullptr;
        sp.num_dests = num_dests;
        sp.pay_in = cur_pay;
        sp.pay_out = pay ? (odd ? b.pay_b : b.pay_a) : nullptr;
        if (i == 0)
            DR_TRY_HIP(dr::launch_radix_validate_hist(dest, num_dests, src_id, src_bound, sp, n, tile_log2, b.hist,
                                                      b.tile_flags, s),
                       "radix histogram launch");
        else
            DR_TRY_HIP(dr::launch_radix_hist(sp, n, tile_log2, b.hist, status, s), "radix histogram launch");
        DR_TRY_HIP(dr::launch_radix_scan(b.hist, b.nblocks, 1 << sp.bits, b.totals, status,
                                         i == 0 ? b.tile_flags : nullptr, s),
                   "radix scan launch");
        DR_TRY_HIP(dr::launch_radix_scatter(sp, n, tile_log2, b.hist, b.totals, status, s), "radix scatter launch");
        cur_dest = sp.dest_out;
        cur_src = sp.src_out;
        cur_val = sp.val_out;
        cur_pay = sp.pay_out;
    }
    if (pay_sorted_out) *pay_sorted_out = cur_pay;
    const bool defer = seg_deferred && !seg_in_scatter;
    if (seg_deferred) *seg_deferred = defer;
    if (sorted_dest_out) *sorted_dest_out = cur_dest;
    if (!seg_in_scatter && !defer)
        DR_TRY_HIP(dr::launch_seg_offsets(cur_dest, n, num_dests, seg_offsets, status, s), "segment offsets launch");
    return DR_OK;
}

// Upper bounds of the index_add plan for tiles of tc = 2^m chunks.
struct PlanBounds {
    int64_t tiles, multis, pslots;
};
PlanBounds plan_bounds(int64_t n, int32_t num_dests, int tc_log2) {
    const int64_t tc = (int64_t)1 << tc_log2;
    const int64_t touched = std::min<int64_t>(num_dests, n);
    PlanBounds b;
    // sum_d ceil(C_d / tc) <= sum_d (C_d / tc + 1), sum_d C_d <= n/8 + touched
    b.tiles = touched + (n / 8 + touched + tc - 1) / tc + 1;
    // a multi-tile segment has more than 8*tc rows
    b.multis = n / (8 * tc) + 1;
    // its tile count is below 2*C_d/tc <= L_d/(4 tc) + 2/tc; summed, <= n/(2 tc)
    b.pslots = n / (2 * tc) + 2;
    return b;
}

struct IndexAddBuffers {
    int32_t* status;
    int32_t* perm;
    int32_t* seg;
    SortBuffers sort;
    int32_t* block_sums;
    dr::TileRec* tiles;
    dr::MultiRec* multis;
    float* partials;
    uint64_t* fp_parts;  // fingerprint changes: segreduce's workgroups, then tilecombine's
};

// The persistent reduce grids hold at most this many workgroups each.
constexpr int64_t kMaxReduceGrid = 65536;

// The sort tile of an index_add: a sort that also moves a payload keeps a
// third array per key in registers and LDS, so its default tile is at most
// 2^12 keys (two workgroups per CU instead of one).
int index_add_sort_tile(const dr::Launch& lc, int64_t n, bool with_pay) {
    const int t = lc.sort_tile(n);
    return with_pay && lc.sort_tile_log2 == 0 && t > 12 ? 12 : t;
}

// with_pay: the formed-contribution path, whose sort also moves the scales
// into sorted order.
IndexAddBuffers carve_index_add(Carver& c, int64_t n, int32_t num_dests, int64_t hidden, bool sort_inside,
                                int tc_log2, int sort_tile_log2, bool with_pay = false) {
    IndexAddBuffers b{};
    b.status = c.take<int32_t>(dr::kStatusBytes / sizeof(int32_t));
    if (sort_inside) {
        b.perm = c.take<int32_t>(n);
        b.seg = c.take<int32_t>((int64_t)num_dests + 1);
        b.sort = carve_sort(c, n, false, sort_tile_log2, with_pay);
    }
    const PlanBounds pb = plan_bounds(n, num_dests, tc_log2);
    b.block_sums = c.take<int32_t>(3 * dr::plan_blocks(num_dests));
    b.tiles = c.take<dr::TileRec>(pb.tiles);
    b.multis = c.take<dr::MultiRec>(pb.multis);
    b.partials = c.take<float>(pb.pslots * hidden);
    b.fp_parts = c.take<uint64_t>(2 * kMaxReduceGrid);
    return b;
}

int elems16(dr_dtype dt) { return dt == DR_BF16 ? 8 : 4; }

dr_status check_dtype(dr_dtype dt, const char* what) {
    if (dt != DR_F32 && dt != DR_BF16) return fail(DR_ERR_UNSUPPORTED, "%s: dtype %d is not fp32 or bf16", what, (int)dt);
    return DR_OK;
}

dr_status check_rows(const void* p, dr_dtype dt, int64_t hidden, const char* what) {
    if (hidden < 1) return fail(DR_ERR_INVALID_ARGUMENT, "%s: hidden must be >= 1 (got %lld)", what, (long long)hidden);
    if (hidden % elems16(dt) != 0)
        return fail(DR_ERR_INVALID_ARGUMENT, "%s: hidden (%lld) must be a multiple of %d for this dtype", what,
                    (long long)hidden, elems16(dt));
    if (p && !aligned(p, 16)) return fail(DR_ERR_INVALID_ARGUMENT, "%s: row data must be 16-byte aligned", what);
    return DR_OK;
}

constexpr int64_t kMaxN = (int64_t)1 << 31;

struct WgradBuffers {
    int32_t* status;
    int32_t* cum_items;
    int32_t* chunk_base;
    float* chunks;
};
WgradBuffers carve_wgrad(Carver& c, int64_t K, int32_t num_groups, int32_t split, int64_t M, int64_t N) {
    WgradBuffers b{};
    b.status = c.take<int32_t>(dr::kStatusBytes / sizeof(int32_t));
    b.cum_items = c.take<int32_t>((int64_t)num_groups + 1);
    b.chunk_base = c.take<int32_t>(num_groups);
    b.chunks = c.take<float>(dr::wgrad_max_chunk_rows(K, split) * M * N);
    return b;
}

}  // namespace

namespace dr {

dr_status report(dr_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return s;
}

dr_status report_ok() { return ok(); }

dr_status report_hip(hipError_t e, const char* what) { return hip_fail(e, what); }

dr_status validate_combine(const char* what, const void* rows, dr_dtype rows_dtype, int64_t num_rows, int64_t hidden,
                           const int32_t* row_of, const float* gates, int64_t T, int32_t k, const float* out,
                           const int32_t* dev_status) {
    dr_status st = check_dtype(rows_dtype, what);
    if (st != DR_OK) return st;
    if ((st = check_rows(rows, rows_dtype, hidden, what)) != DR_OK) return st;
    if (!aligned(out, 16)) return fail(DR_ERR_INVALID_ARGUMENT, "%s: out must be 16-byte aligned", what);
    if (T < 0 || num_rows < 0 || num_rows >= kMaxN) return fail(DR_ERR_INVALID_ARGUMENT, "%s: bad T or num_rows", what);
    if (k < 1) return fail(DR_ERR_INVALID_ARGUMENT, "%s: k must be >= 1", what);
    if (k > 64) return fail(DR_ERR_UNSUPPORTED, "%s: k = %d > 64 is not supported", what, k);
    if (T > 0 && (!rows || !row_of || !gates || !out)) return fail(DR_ERR_INVALID_ARGUMENT, "%s: null pointer", what);
    if (T > 0 && (!aligned(row_of, 4) || !aligned(gates, 4)))
        return fail(DR_ERR_INVALID_ARGUMENT, "%s: row_of/gates must be 4-byte aligned", what);
    if (dev_status && !aligned(dev_status, 4)) return fail(DR_ERR_INVALID_ARGUMENT, "%s: misaligned dev_status", what);
    if (T * ((hidden / elems16(rows_dtype) + 63) / 64) >= ((int64_t)1 << 32))
        return fail(DR_ERR_UNSUPPORTED, "%s: T * column slices must be below 2^32", what);
    return DR_OK;
}

Launch launch_config() {
    Launch l;
    l.grid_blocks = g_params.grid_blocks;
    l.tile_chunks_log2 = g_params.tile_chunks_log2 ? g_params.tile_chunks_log2 : kDefaultTileChunksLog2;
    l.sort_tile_log2 = g_params.sort_tile_log2;
    l.chunks_in_flight = g_params.chunks_in_flight ? g_params.chunks_in_flight : 1;
    l.splitk_stream = g_params.splitk_stream != 2;
    return l;
}

int device_cu_count() {
    // per device, filled on first use; atomic because any host thread may launch
    constexpr int kSlots = 256;
    static std::atomic<int> cache[kSlots];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    if (dev < kSlots) {
        const int known = cache[dev].load(std::memory_order_relaxed);
        if (known > 0) return known;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    if (dev < kSlots) cache[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

}  // namespace dr

extern "C" {

const char* dr_status_string(dr_status s) {
    switch (s) {
        case DR_OK: return "DR_OK";
        case DR_ERR_INVALID_ARGUMENT: return "DR_ERR_INVALID_ARGUMENT";
        case DR_ERR_UNSUPPORTED: return "DR_ERR_UNSUPPORTED";
        case DR_ERR_WORKSPACE_TOO_SMALL: return "DR_ERR_WORKSPACE_TOO_SMALL";
        case DR_ERR_INDEX_OUT_OF_RANGE: return "DR_ERR_INDEX_OUT_OF_RANGE";
        case DR_ERR_HIP: return "DR_ERR_HIP";
        case DR_ERR_BAD_PLAN: return "DR_ERR_BAD_PLAN";
    }
    return "DR_ERR_UNKNOWN";
}

const char* dr_last_error(void) { return g_err.c_str(); }

int32_t dr_version(void) { return 101; }

dr_status dr_set_phase_events(hipEvent_t reduce_begin, hipEvent_t reduce_end) {
    if ((reduce_begin == nullptr) != (reduce_end == nullptr))
        return fail(DR_ERR_INVALID_ARGUMENT, "dr_set_phase_events: give both events or neither");
    g_reduce_begin = reduce_begin;
    g_reduce_end = reduce_end;
    return ok();
}

dr_status dr_set_launch_params(const dr_launch_params* p) {
    if (!p) {
        g_params = dr_launch_params{0, 0, 0, 0, 0};
        return ok();
    }
    if (p->grid_blocks < 0 || p->grid_blocks > 65536)
        return fail(DR_ERR_INVALID_ARGUMENT, "grid_blocks must be 0 or 1..65536");
    if (p->tile_chunks_log2 != 0 &&
        (p->tile_chunks_log2 < dr::kMinTileChunksLog2 || p->tile_chunks_log2 > dr::kMaxTileChunksLog2))
        return fail(DR_ERR_INVALID_ARGUMENT, "tile_chunks_log2 must be 0 or %d..%d", dr::kMinTileChunksLog2,
                    dr::kMaxTileChunksLog2);
    if (p->sort_tile_log2 != 0 &&
        (p->sort_tile_log2 < dr::kMinSortTileLog2 || p->sort_tile_log2 > dr::kMaxSortTileLog2))
        return fail(DR_ERR_INVALID_ARGUMENT, "sort_tile_log2 must be 0 or %d..%d", dr::kMinSortTileLog2,
                    dr::kMaxSortTileLog2);
    if (p->chunks_in_flight != 0 && p->chunks_in_flight != 1 && p->chunks_in_flight != 2)
        return fail(DR_ERR_INVALID_ARGUMENT, "chunks_in_flight must be 0, 1 or 2");
    if (p->splitk_stream < 0 || p->splitk_stream > 2)
        return fail(DR_ERR_INVALID_ARGUMENT, "splitk_stream must be 0, 1 or 2");
    g_params = *p;
    return ok();
}

// ---------------------------------------------------------------------------
size_t dr_sort_workspace_size(int64_t n, int32_t num_dests, int32_t src_id_bound) {
    (void)num_dests;
    Carver c(nullptr);
    c.take<int32_t>(dr::kStatusBytes / sizeof(int32_t));
    carve_sort(c, n < 0 ? 0 : n, src_id_bound > 0, dr::launch_config().sort_tile(n));
    return c.off;
}

dr_status dr_sort_by_dest(const int32_t* dest, const int32_t* src_id, int32_t src_id_bound, int64_t n,
                          int32_t num_dests, int32_t* perm, int32_t* seg_offsets, int32_t* inv_perm, void* ws,
                          size_t ws_bytes, hipStream_t stream) {
    const char* what = "dr_sort_by_dest";
    if (n < 0 || n >= kMaxN) return fail(DR_ERR_INVALID_ARGUMENT, "%s: n must be in [0, 2^31)", what);
    if (num_dests < 1) return fail(DR_ERR_INVALID_ARGUMENT, "%s: num_dests must be >= 1", what);
    if (src_id && src_id_bound < 1) return fail(DR_ERR_INVALID_ARGUMENT, "%s: src_id_bound must be >= 1", what);
    if (n > 0 && (!dest || !perm)) return fail(DR_ERR_INVALID_ARGUMENT, "%s: null dest or perm", what);
    if (!seg_offsets || !ws) return fail(DR_ERR_INVALID_ARGUMENT, "%s: null seg_offsets or workspace", what);
    if (!aligned(ws, 16)) return fail(DR_ERR_INVALID_ARGUMENT, "%s: workspace must be 16-byte aligned", what);
    const int tile_log2 = dr::launch_config().sort_tile(n);
    Carver c(ws);
    int32_t* status = c.take<int32_t>(dr::kStatusBytes / sizeof(int32_t));
    const SortBuffers b = carve_sort(c, n, src_id != nullptr, tile_log2);
    if (c.off > ws_bytes)
        return fail(DR_ERR_WORKSPACE_TOO_SMALL, "%s: workspace has %zu bytes, needs %zu", what, ws_bytes, c.off);
    const dr_status st = run_sort(dest, src_id, src_id_bound, n, num_dests, perm, seg_offsets, inv_perm, status, b,
                                  tile_log2, stream);
    return st == DR_OK ? ok() : st;
}

// ---------------------------------------------------------------------------
dr_status dr_combine(const void* rows, dr_dtype rows_dtype, int64_t num_rows, int64_t hidden,
                     const int32_t* row_of, const float* gates, int64_t T, int32_t k, float* out,
                     int32_t* dev_status, hipStream_t stream) {
    const dr_status st = dr::validate_combine("dr_combine", rows, rows_dtype, num_rows, hidden, row_of, gates, T, k,
                                              out, dev_status);
    if (st != DR_OK) return st;
    DR_TRY_HIP(dr::launch_combine(rows, rows_dtype, num_rows, hidden, row_of, gates, T, k, out, dev_status, false,
                                  nullptr, stream),
               "combine launch");
    return ok();
}

size_t dr_combine_fingerprinted_workspace_size(dr_dtype rows_dtype, int64_t hidden, int64_t T) {
    if (hidden < 1 || T < 0) return dr::kStatusBytes;
    const int64_t nb = dr::combine_fp_blocks(rows_dtype, hidden, T, 64);  // the largest count over k
    return dr::kStatusBytes + align_up((size_t)nb * sizeof(uint64_t)) +
           align_up((size_t)dr::fingerprint_group_count(nb) * sizeof(uint64_t));
}

dr_status dr_combine_fingerprinted(const void* rows, dr_dtype rows_dtype, int64_t num_rows, int64_t hidden,
                                   const int32_t* row_of, const float* gates, int64_t T, int32_t k, float* out,
                                   uint64_t* out_hash, void* ws, size_t ws_bytes, int32_t* dev_status,
                                   hipStream_t stream) {
    const char* what = "dr_combine_fingerprinted";
    const dr_status st = dr::validate_combine(what, rows, rows_dtype, num_rows, hidden, row_of, gates, T, k, out,
                                              dev_status);
    if (st != DR_OK) return st;
    if (!out_hash || !aligned(out_hash, 8)) return fail(DR_ERR_INVALID_ARGUMENT, "%s: bad out_hash", what);
    if (!ws || !aligned(ws, 16)) return fail(DR_ERR_INVALID_ARGUMENT, "%s: bad workspace", what);
    if (ws_bytes < dr_combine_fingerprinted_workspace_size(rows_dtype, hidden, T))
        return fail(DR_ERR_WORKSPACE_TOO_SMALL, "%s: workspace has %zu bytes, needs %zu", what, ws_bytes,
                    dr_combine_fingerprinted_workspace_size(rows_dtype, hidden, T));
    const int64_t nb_max = dr::combine_fp_blocks(rows_dtype, hidden, T, 64);
    const int64_t nb = dr::combine_fp_blocks(rows_dtype, hidden, T, k);
    Carver c(ws);
    c.take<uint8_t>(dr::kStatusBytes);
    uint64_t* partials = c.take<uint64_t>(nb_max);
    uint64_t* group_sums = c.take<uint64_t>(dr::fingerprint_group_count(nb_max));
    DR_TRY_HIP(dr::launch_combine(rows, rows_dtype, num_rows, hidden, row_of, gates, T, k, out, dev_status, false,
                                  partials, stream),
               "combine launch");
    DR_TRY_HIP(dr::launch_fingerprint_final(partials, nb, T * hidden * (int64_t)sizeof(float), out_hash, group_sums,
                                            stream),
               "fingerprint launch");
    return ok();
}

dr_status dr_combine_atomic(const void* rows, dr_dtype rows_dtype, int64_t num_rows, int64_t hidden,
                            const int32_t* row_of, const float* gates, int64_t T, int32_t k, float* out,
                            int32_t* dev_status, hipStream_t stream) {
    const char* what = "dr_combine_atomic";
    dr_status st = check_dtype(rows_dtype, what);
    if (st != DR_OK) return st;
    if ((st = check_rows(rows, rows_dtype, hidden, what)) != DR_OK) return st;
    if (!aligned(out, 16)) return fail(DR_ERR_INVALID_ARGUMENT, "%s: out must be 16-byte aligned", what);
    if (T < 0 || num_rows < 0 || num_rows >= kMaxN) return fail(DR_ERR_INVALID_ARGUMENT, "%s: bad T or num_rows", what);
    if (k < 1 || k > 64) return fail(DR_ERR_UNSUPPORTED, "%s: k must be in [1, 64]", what);
    if (T > 0 && (!rows || !row_of || !gates || !out)) return fail(DR_ERR_INVALID_ARGUMENT, "%s: null pointer", what);
    if (T * k * ((hidden / elems16(rows_dtype) + 63) / 64) >= ((int64_t)1 << 32))
        return fail(DR_ERR_UNSUPPORTED, "%s: T * k * column slices must be below 2^32", what);
    DR_TRY_HIP(dr::launch_combine(rows, rows_dtype, num_rows, hidden, row_of, gates, T, k, out, dev_status, true,
                                  nullptr, stream),
               "combine_atomic launch");
    return ok();
}

// ---------------------------------------------------------------------------
size_t dr_index_add_workspace_size(int64_t n, int32_t num_dests, int64_t hidden) {
    const dr::Launch lc = dr::launch_config();
    Carver c(nullptr);
    carve_index_add(c, n < 0 ? 0 : n, num_dests < 1 ? 1 : num_dests, hidden < 1 ? 1 : hidden, true,
                    lc.tile_chunks_log2, lc.sort_tile(n));
    return c.off;
}

namespace {

// The contributions of an index_add: rows of src, or (scale != null) the
// rows fl32(scale[p] * src[p / rows_per_src]) formed in the reduce kernel.
struct Contributions {
    const void* src;
    dr_dtype dtype;
    const float* scale;
    int32_t rows_per_src;
};

dr_status run_index_add(const char* what, float* out, int32_t num_dests, int64_t hidden, const Contributions& c,
                        int64_t n, const int32_t* index, const int32_t* perm, const int32_t* seg_offsets, void* ws,
                        size_t ws_bytes, uint64_t* inout_hash, hipStream_t stream) {
    if (!out || !aligned(out, 16)) return fail(DR_ERR_INVALID_ARGUMENT, "%s: out must be non-null and 16-byte aligned", what);
    if (num_dests < 1) return fail(DR_ERR_INVALID_ARGUMENT, "%s: num_dests must be >= 1", what);
    if (n < 0 || n >= kMaxN) return fail(DR_ERR_INVALID_ARGUMENT, "%s: n must be in [0, 2^31)", what);
    if (n > 0 && (!c.src || !index)) return fail(DR_ERR_INVALID_ARGUMENT, "%s: null source rows or index", what);
    if ((perm == nullptr) != (seg_offsets == nullptr))
        return fail(DR_ERR_INVALID_ARGUMENT, "%s: perm and seg_offsets must both be given or both be NULL", what);
    if (!ws || !aligned(ws, 16)) return fail(DR_ERR_INVALID_ARGUMENT, "%s: workspace must be non-null, 16-byte aligned", what);
    const dr::Launch lc = dr::launch_config();
    const bool sort_inside = perm == nullptr;
    {
        // the reduce kernels index (tile, column slice) work items with 32 bits
        const PlanBounds pb = plan_bounds(n, num_dests, lc.tile_chunks_log2);
        const int64_t slices = (hidden / 4 + 15) / 16;  // upper bound over both dtypes and group sizes
        if (pb.tiles * slices >= ((int64_t)1 << 32))
            return fail(DR_ERR_UNSUPPORTED, "%s: n and hidden too large for one call", what);
    }
    Carver cv(ws);
    const int sort_tile = index_add_sort_tile(lc, n, c.scale != nullptr);
    const IndexAddBuffers b = carve_index_add(cv, n, num_dests, hidden, sort_inside, lc.tile_chunks_log2,
                                              sort_tile, c.scale != nullptr);
    if (cv.off > ws_bytes)
        return fail(DR_ERR_WORKSPACE_TOO_SMALL, "%s: workspace has %zu bytes, needs %zu", what, ws_bytes, cv.off);
    const int32_t* p = perm;
    const int32_t* seg = seg_offsets;
    bool seg_deferred = false;  // the plan count then also finds the segment offsets
    const int32_t* sorted_dest = nullptr;
    // Formed contributions read their scale at each sorted position.  When
    // the sort runs here the scales travel with the keys (read in input
    // order, written in sorted order), so the reduce reads them contiguously
    // instead of one scattered 4-byte load (a whole cache line) per row.
    const float* scale = c.scale;
    bool scale_sorted = false;
    if (sort_inside) {
        // the sort writes the status word
        const dr_status st = run_sort(index, nullptr, 0, n, num_dests, b.perm, b.seg, nullptr, b.status, b.sort,
                                      sort_tile, stream, &seg_deferred, &sorted_dest, c.scale,
                                      c.scale ? &scale : nullptr);
        if (st != DR_OK) return st;
        scale_sorted = c.scale != nullptr && n > 0;
        if (c.scale && n == 0) scale = c.scale;
        p = b.perm;
        seg = b.seg;
    } else {
        DR_TRY_HIP(dr::launch_fill_status(b.status, stream), "status reset launch");
        DR_TRY_HIP(dr::launch_plan_validate(perm, seg_offsets, index, n, num_dests, b.status, stream),
                   "plan validation launch");
    }
    if (seg_deferred)
        DR_TRY_HIP(dr::launch_plan_count_search(sorted_dest, n, num_dests, lc.tile_chunks_log2, b.seg, b.block_sums,
                                                b.status, stream),
                   "plan count launch");
    else
        DR_TRY_HIP(dr::launch_plan_count(seg, num_dests, n, lc.tile_chunks_log2, b.block_sums, b.status, stream),
                   "plan count launch");
    DR_TRY_HIP(dr::launch_plan_write(seg, num_dests, lc.tile_chunks_log2, b.block_sums, b.tiles, b.multis, b.status,
                                     stream),
               "plan write launch");
    const int64_t grid = dr::persistent_grid();
    uint64_t* fp_seg = inout_hash ? b.fp_parts : nullptr;
    uint64_t* fp_tc = inout_hash ? b.fp_parts + grid : nullptr;
    if (g_reduce_begin) DR_TRY_HIP(hipEventRecord(g_reduce_begin, stream), "phase event");
    DR_TRY_HIP(dr::launch_segreduce(out, hidden, c.src, c.dtype, n, p, b.tiles, b.partials, lc.tile_chunks_log2,
                                    lc.chunks_in_flight, scale, scale_sorted, c.rows_per_src, b.status, fp_seg,
                                    stream),
               "segmented reduce launch");
    DR_TRY_HIP(dr::launch_tilecombine(out, hidden, b.partials, b.multis, n, lc.tile_chunks_log2, b.status, fp_tc,
                                      stream),
               "tile combine launch");
    if (g_reduce_end) DR_TRY_HIP(hipEventRecord(g_reduce_end, stream), "phase event");
    if (inout_hash)
        DR_TRY_HIP(dr::launch_fingerprint_update(b.fp_parts, 2 * grid, b.status, inout_hash, stream),
                   "fingerprint update launch");
    return ok();
}

}  // namespace

dr_status dr_index_add(float* out, int32_t num_dests, int64_t hidden, const void* src, dr_dtype src_dtype, int64_t n,
                       const int32_t* index, const int32_t* perm, const int32_t* seg_offsets, void* ws,
                       size_t ws_bytes, hipStream_t stream) {
    const char* what = "dr_index_add";
    dr_status st = check_dtype(src_dtype, what);
    if (st != DR_OK) return st;
    if ((st = check_rows(src, src_dtype, hidden, what)) != DR_OK) return st;
    return run_index_add(what, out, num_dests, hidden, Contributions{src, src_dtype, nullptr, 1}, n, index, perm,
                         seg_offsets, ws, ws_bytes, nullptr, stream);
}

dr_status dr_index_add_fingerprinted(float* out, int32_t num_dests, int64_t hidden, const void* src,
                                     dr_dtype src_dtype, int64_t n, const int32_t* index, const int32_t* perm,
                                     const int32_t* seg_offsets, uint64_t* inout_hash, void* ws, size_t ws_bytes,
                                     hipStream_t stream) {
    const char* what = "dr_index_add_fingerprinted";
    dr_status st = check_dtype(src_dtype, what);
    if (st != DR_OK) return st;
    if ((st = check_rows(src, src_dtype, hidden, what)) != DR_OK) return st;
    if (!inout_hash || !aligned(inout_hash, 8))
        return fail(DR_ERR_INVALID_ARGUMENT, "%s: inout_hash must be a non-null, 8-byte aligned device pointer", what);
    return run_index_add(what, out, num_dests, hidden, Contributions{src, src_dtype, nullptr, 1}, n, index, perm,
                         seg_offsets, ws, ws_bytes, inout_hash, stream);
}

size_t dr_sparse_attn_dk_workspace_size(int64_t num_queries, int32_t topk, int32_t num_keys, int64_t head_dim) {
    const int64_t n = num_queries < 0 || topk < 1 ? 0 : num_queries * (int64_t)topk;
    const dr::Launch lc = dr::launch_config();
    Carver c(nullptr);
    carve_index_add(c, n, num_keys < 1 ? 1 : num_keys, head_dim < 1 ? 1 : head_dim, true, lc.tile_chunks_log2,
                    index_add_sort_tile(lc, n, true), true);
    return c.off;
}

dr_status dr_sparse_attn_dk(float* dK, int32_t num_keys, int64_t head_dim, const void* Q, dr_dtype q_dtype,
                            const float* dS, const int32_t* key_idx, int64_t num_queries, int32_t topk,
                            const int32_t* perm, const int32_t* seg_offsets, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
    const char* what = "dr_sparse_attn_dk";
    dr_status st = check_dtype(q_dtype, what);
    if (st != DR_OK) return st;
    if ((st = check_rows(Q, q_dtype, head_dim, what)) != DR_OK) return st;
    if (num_queries < 0 || topk < 1)
        return fail(DR_ERR_INVALID_ARGUMENT, "%s: num_queries must be >= 0 and topk >= 1", what);
    if (num_queries > kMaxN / topk)
        return fail(DR_ERR_INVALID_ARGUMENT, "%s: num_queries * topk must be below 2^31", what);
    const int64_t n = num_queries * (int64_t)topk;
    if (n > 0 && (!dS || !aligned(dS, 4))) return fail(DR_ERR_INVALID_ARGUMENT, "%s: dS must be non-null and 4-byte aligned", what);
    return run_index_add(what, dK, num_keys, head_dim, Contributions{Q, q_dtype, dS, topk}, n, key_idx, perm,
                         seg_offsets, ws, ws_bytes, nullptr, stream);
}

dr_status dr_index_add_atomic(float* out, int32_t num_dests, int64_t hidden, const void* src, dr_dtype src_dtype,
                              int64_t n, const int32_t* index, int32_t* dev_status, hipStream_t stream) {
    const char* what = "dr_index_add_atomic";
    dr_status st = check_dtype(src_dtype, what);
    if (st != DR_OK) return st;
    if ((st = check_rows(src, src_dtype, hidden, what)) != DR_OK) return st;
    if (!out || !aligned(out, 16)) return fail(DR_ERR_INVALID_ARGUMENT, "%s: out must be non-null and 16-byte aligned", what);
    if (num_dests < 1 || n < 0 || n >= kMaxN) return fail(DR_ERR_INVALID_ARGUMENT, "%s: bad num_dests or n", what);
    if (n > 0 && (!src || !index)) return fail(DR_ERR_INVALID_ARGUMENT, "%s: null src or index", what);
    if (n * (hidden / elems16(src_dtype)) >= ((int64_t)1 << 32))
        return fail(DR_ERR_UNSUPPORTED, "%s: n * hidden too large for one call", what);
    DR_TRY_HIP(dr::launch_index_add_atomic(out, num_dests, hidden, src, src_dtype, n, index, dev_status, stream),
               "index_add_atomic launch");
    return ok();
}

// ---------------------------------------------------------------------------
static dr_status check_splitk(const void* X, const void* dY, int64_t K, int64_t M, int64_t N, int32_t splits,
                              const void* out, const char* what) {
    if (!X || !dY || !out) return fail(DR_ERR_INVALID_ARGUMENT, "%s: null pointer", what);
    if (K < 1 || M < 1 || N < 1) return fail(DR_ERR_INVALID_ARGUMENT, "%s: K, M, N must be >= 1", what);
    if (splits < 1 || splits > 65535) return fail(DR_ERR_INVALID_ARGUMENT, "%s: splits must be in [1, 65535]", what);
    const int64_t kc = (K + splits - 1) / splits;
    if ((int64_t)(splits - 1) * kc >= K)
        return fail(DR_ERR_INVALID_ARGUMENT, "%s: %d splits of %lld tokens leave an empty split (K = %lld)", what, splits,
                    (long long)kc, (long long)K);
    if (!aligned(X, 16) || !aligned(dY, 2) || !aligned(out, 4))
        return fail(DR_ERR_INVALID_ARGUMENT, "%s: X must be 16-byte aligned", what);
    // (split, N tile, M tile) items are counted in 32 bits on the device
    if ((M + 63) / 64 > 0x7FFFFFFF || (N + 31) / 32 > 0x7FFFFFFF ||
        ((M + 63) / 64) * ((N + 31) / 32) > 0x7FFFFFFF / splits)
        return fail(DR_ERR_UNSUPPORTED, "%s: M, N and splits give too many tiles for one launch", what);
    return DR_OK;
}

dr_status dr_splitk_gemm_tn(const void* X, const void* dY, int64_t K, int64_t M, int64_t N, int32_t splits,
                            float* partials, hipStream_t stream) {
    const dr_status st = check_splitk(X, dY, K, M, N, splits, partials, "dr_splitk_gemm_tn");
    if (st != DR_OK) return st;
    DR_TRY_HIP(dr::launch_splitk_gemm(static_cast<const uint16_t*>(X), static_cast<const uint16_t*>(dY), K, M, N,
                                      splits, partials, false, stream),
               "split-K GEMM launch");
    return ok();
}

dr_status dr_splitk_gemm_tn_atomic(const void* X, const void* dY, int64_t K, int64_t M, int64_t N, int32_t splits,
                                   float* out, hipStream_t stream) {
    const dr_status st = check_splitk(X, dY, K, M, N, splits, out, "dr_splitk_gemm_tn_atomic");
    if (st != DR_OK) return st;
    DR_TRY_HIP(dr::launch_splitk_gemm(static_cast<const uint16_t*>(X), static_cast<const uint16_t*>(dY), K, M, N,
                                      splits, out, true, stream),
               "split-K atomic GEMM launch");
    return ok();
}

dr_status dr_splitk_reduce(const float* partials, int32_t splits, int64_t count, float* out, hipStream_t stream) {
    const char* what = "dr_splitk_reduce";
    if (splits < 1) return fail(DR_ERR_INVALID_ARGUMENT, "%s: splits must be >= 1", what);
    if (count < 0) return fail(DR_ERR_INVALID_ARGUMENT, "%s: count must be >= 0", what);
    if (count > 0 && (!partials || !out)) return fail(DR_ERR_INVALID_ARGUMENT, "%s: null pointer", what);
    if (count > 0 && (!aligned(partials, 16) || !aligned(out, 16)))
        return fail(DR_ERR_INVALID_ARGUMENT, "%s: partials and out must be 16-byte aligned", what);
    if (splits >= (1 << 27)) return fail(DR_ERR_UNSUPPORTED, "%s: too many splits", what);
    DR_TRY_HIP(dr::launch_splitk_reduce(partials, splits, count, out, nullptr, stream), "split reduce launch");
    return ok();
}

size_t dr_splitk_reduce_fingerprinted_workspace_size(int32_t splits, int64_t count) {
    if (splits < 1 || count < 0) return dr_fingerprint_workspace_size(0);
    const int64_t nb = dr::splitk_reduce_blocks(splits, count);
    const size_t fused = dr::kStatusBytes + align_up((size_t)nb * sizeof(uint64_t)) +
                         align_up((size_t)dr::fingerprint_group_count(nb) * sizeof(uint64_t));
    const size_t separate = dr_fingerprint_workspace_size(count * (int64_t)sizeof(float));
    return fused > separate ? fused : separate;
}

dr_status dr_splitk_reduce_fingerprinted(const float* partials, int32_t splits, int64_t count, float* out,
                                         uint64_t* out_hash, void* ws, size_t ws_bytes, hipStream_t stream) {
    const char* what = "dr_splitk_reduce_fingerprinted";
    if (splits < 1) return fail(DR_ERR_INVALID_ARGUMENT, "%s: splits must be >= 1", what);
    if (count < 0) return fail(DR_ERR_INVALID_ARGUMENT, "%s: count must be >= 0", what);
    if (count > 0 && (!partials || !out)) return fail(DR_ERR_INVALID_ARGUMENT, "%s: null pointer", what);
    if (count > 0 && (!aligned(partials, 16) || !aligned(out, 16)))
        return fail(DR_ERR_INVALID_ARGUMENT, "%s: partials and out must be 16-byte aligned", what);
    if (splits >= (1 << 27)) return fail(DR_ERR_UNSUPPORTED, "%s: too many splits", what);
    if (!out_hash || !aligned(out_hash, 8)) return fail(DR_ERR_INVALID_ARGUMENT, "%s: bad out_hash", what);
    if (!ws || !aligned(ws, 16)) return fail(DR_ERR_INVALID_ARGUMENT, "%s: bad workspace", what);
    const size_t need = dr_splitk_reduce_fingerprinted_workspace_size(splits, count);
    if (ws_bytes < need)
        return fail(DR_ERR_WORKSPACE_TOO_SMALL, "%s: workspace has %zu bytes, needs %zu", what, ws_bytes, need);
    const int64_t nbytes = count * (int64_t)sizeof(float);
    if (count % 4 != 0) {
        // pieces of 16 bytes are what the reduce hashes as it stores; otherwise hash out afterwards
        DR_TRY_HIP(dr::launch_splitk_reduce(partials, splits, count, out, nullptr, stream), "split reduce launch");
        uint64_t* parts = reinterpret_cast<uint64_t*>(static_cast<char*>(ws) + dr::kStatusBytes);
        DR_TRY_HIP(dr::launch_fingerprint(out, nbytes, out_hash, parts, stream), "fingerprint launch");
        return ok();
    }
    const int64_t nb = dr::splitk_reduce_blocks(splits, count);
    Carver c(ws);
    c.take<uint8_t>(dr::kStatusBytes);
    uint64_t* parts = c.take<uint64_t>(nb);
    uint64_t* group_sums = c.take<uint64_t>(dr::fingerprint_group_count(nb));
    DR_TRY_HIP(dr::launch_splitk_reduce(partials, splits, count, out, parts, stream), "split reduce launch");
    DR_TRY_HIP(dr::launch_fingerprint_final(parts, nb, nbytes, out_hash, group_sums, stream), "fingerprint launch");
    return ok();
}

// ---------------------------------------------------------------------------
int64_t dr_grouped_splitk_max_slots(int64_t K, int32_t num_groups, int32_t split_tokens) {
    if (K < 0 || num_groups < 1 || split_tokens < 1) return 0;
    // sum_g ceil(c_g / s) <= sum_g (c_g / s + 1) <= K / s + G
    return K / split_tokens + num_groups;
}

size_t dr_grouped_splitk_workspace_size(int64_t K, int32_t num_groups, int32_t split_tokens) {
    Carver c(nullptr);
    c.take<int32_t>(dr::kStatusBytes / sizeof(int32_t));
    c.take<int2>(dr_grouped_splitk_max_slots(K, num_groups, split_tokens));
    return c.off;
}

dr_status dr_grouped_splitk_gemm_tn(const void* X, const void* dY, int64_t K, int64_t M, int64_t N,
                                    const int32_t* group_offsets, int32_t num_groups, int32_t split_tokens,
                                    float* partials, int64_t partial_slots, int32_t* slot_offsets, void* ws,
                                    size_t ws_bytes, hipStream_t stream) {
    const char* what = "dr_grouped_splitk_gemm_tn";
    if (!X || !dY || !partials || !group_offsets || !slot_offsets || !ws)
        return fail(DR_ERR_INVALID_ARGUMENT, "%s: null pointer", what);
    if (K < 1 || M < 1 || N < 1) return fail(DR_ERR_INVALID_ARGUMENT, "%s: K, M, N must be >= 1", what);
    if (num_groups < 1 || num_groups > 65535)
        return fail(DR_ERR_INVALID_ARGUMENT, "%s: num_groups must be in [1, 65535]", what);
    if (split_tokens < 1) return fail(DR_ERR_INVALID_ARGUMENT, "%s: split_tokens must be >= 1", what);
    // token indices and slot ranges are int32 on the device
    if (K >= kMaxN - split_tokens) return fail(DR_ERR_UNSUPPORTED, "%s: K too large for one call", what);
    if (!aligned(X, 16) || !aligned(dY, 2) || !aligned(partials, 4) || !aligned(group_offsets, 4) ||
        !aligned(slot_offsets, 4) || !aligned(ws, 16))
        return fail(DR_ERR_INVALID_ARGUMENT, "%s: X and ws must be 16-byte aligned, the rest element-aligned", what);
    const int64_t max_slots = dr_grouped_splitk_max_slots(K, num_groups, split_tokens);
    if (partial_slots < max_slots)
        return fail(DR_ERR_WORKSPACE_TOO_SMALL, "%s: partials hold %lld slots, need %lld", what,
                    (long long)partial_slots, (long long)max_slots);
    if (((M + 63) / 64) * ((N + 31) / 32) > 0x7FFFFFFF / max_slots)
        return fail(DR_ERR_UNSUPPORTED, "%s: M, N and the slot bound give too many tiles for one launch", what);
    if (ws_bytes < dr_grouped_splitk_workspace_size(K, num_groups, split_tokens))
        return fail(DR_ERR_WORKSPACE_TOO_SMALL, "%s: workspace has %zu bytes, needs %zu", what, ws_bytes,
                    dr_grouped_splitk_workspace_size(K, num_groups, split_tokens));
    Carver c(ws);
    int32_t* status = c.take<int32_t>(dr::kStatusBytes / sizeof(int32_t));
    int2* ranges = c.take<int2>(max_slots);
    DR_TRY_HIP(dr::launch_grouped_splitk_gemm(static_cast<const uint16_t*>(X), static_cast<const uint16_t*>(dY), K,
                                              M, N, group_offsets, num_groups, split_tokens, max_slots, slot_offsets,
                                              ranges, status, partials, stream),
               "grouped split-K launch");
    return ok();
}

dr_status dr_grouped_splitk_reduce(const float* partials, int64_t partial_slots, const int32_t* slot_offsets,
                                   int32_t num_groups, int64_t count, float* out, const void* ws,
                                   hipStream_t stream) {
    const char* what = "dr_grouped_splitk_reduce";
    if (!partials || !slot_offsets || !out || !ws) return fail(DR_ERR_INVALID_ARGUMENT, "%s: null pointer", what);
    if (num_groups < 1 || num_groups > 65535)
        return fail(DR_ERR_INVALID_ARGUMENT, "%s: num_groups must be in [1, 65535]", what);
    if (count < 0 || partial_slots < 0) return fail(DR_ERR_INVALID_ARGUMENT, "%s: negative size", what);
    if (!aligned(partials, 4) || !aligned(out, 4) || !aligned(ws, 16))
        return fail(DR_ERR_INVALID_ARGUMENT, "%s: misaligned pointer", what);
    if ((count % 4 == 0) && (!aligned(partials, 16) || !aligned(out, 16)))
        return fail(DR_ERR_INVALID_ARGUMENT, "%s: partials and out must be 16-byte aligned", what);
    DR_TRY_HIP(dr::launch_grouped_reduce(partials, slot_offsets, partial_slots, num_groups, count, out,
                                         static_cast<const int32_t*>(ws), stream),
               "grouped reduce launch");
    return ok();
}

// ---------------------------------------------------------------------------

size_t dr_grouped_wgrad_workspace_size(int64_t K, int32_t num_groups, int32_t split_tokens, int64_t M, int64_t N) {
    if (K < 0 || num_groups < 1 || split_tokens < 1 || M < 1 || N < 1) return 0;
    Carver c(nullptr);
    carve_wgrad(c, K, num_groups, split_tokens, M, N);
    return c.off;
}

dr_status dr_grouped_wgrad(const void* X, const void* dY, int64_t K, int64_t M, int64_t N,
                           const int32_t* group_offsets, int32_t num_groups, int32_t split_tokens, float* out,
                           void* ws, size_t ws_bytes, hipStream_t stream) {
    const char* what = "dr_grouped_wgrad";
    if (!X || !dY || !group_offsets || !out || !ws) return fail(DR_ERR_INVALID_ARGUMENT, "%s: null pointer", what);
    if (K < 1 || M < 1 || N < 1) return fail(DR_ERR_INVALID_ARGUMENT, "%s: K, M, N must be >= 1", what);
    if (num_groups < 1 || num_groups > 65535)
        return fail(DR_ERR_INVALID_ARGUMENT, "%s: num_groups must be in [1, 65535]", what);
    if (split_tokens < 1) return fail(DR_ERR_INVALID_ARGUMENT, "%s: split_tokens must be >= 1", what);
    if (M % 8 != 0 || N % 8 != 0)
        return fail(DR_ERR_UNSUPPORTED, "%s: M and N must be multiples of 8 (the thin split handles other shapes)",
                    what);
    if (!aligned(X, 16) || !aligned(dY, 16) || !aligned(out, 16) || !aligned(group_offsets, 4) || !aligned(ws, 16))
        return fail(DR_ERR_INVALID_ARGUMENT, "%s: X, dY, out and ws must be 16-byte aligned", what);
    // a stage's buffer range (64 token rows) is a 32-bit byte count
    if (M > ((int64_t)1 << 23) || N > ((int64_t)1 << 23))
        return fail(DR_ERR_UNSUPPORTED, "%s: M and N must be at most 2^23", what);
    // token indices are int32 on the device; work items are counted in 31 bits
    if (K >= kMaxN - split_tokens) return fail(DR_ERR_UNSUPPORTED, "%s: K too large for one call", what);
    if (dr::wgrad_max_items(K, num_groups, split_tokens, M, N) >= ((int64_t)1 << 31))
        return fail(DR_ERR_UNSUPPORTED, "%s: M, N and the chunk bound give too many tiles for one call", what);
    if (dr::wgrad_max_chunk_rows(K, split_tokens) >= ((int64_t)1 << 31))
        return fail(DR_ERR_UNSUPPORTED, "%s: too many chunks for one call", what);
    Carver c(ws);
    const WgradBuffers b = carve_wgrad(c, K, num_groups, split_tokens, M, N);
    if (c.off > ws_bytes)
        return fail(DR_ERR_WORKSPACE_TOO_SMALL, "%s: workspace has %zu bytes, needs %zu", what, ws_bytes, c.off);
    DR_TRY_HIP(dr::launch_wgrad(static_cast<const uint16_t*>(X), static_cast<const uint16_t*>(dY), K, M, N,
                                group_offsets, num_groups, split_tokens, out, b.status, b.cum_items, b.chunk_base,
                                b.chunks, stream),
               "grouped wgrad launch");
    return ok();
}

// ---------------------------------------------------------------------------
dr_status dr_permute_rows(const void* rows, int64_t row_bytes, int64_t num_rows, const int32_t* perm,
                          const int32_t* inv_perm, int64_t n, int32_t k, void* out, int32_t* dev_status,
                          hipStream_t stream) {
    const char* what = "dr_permute_rows";
    if (n < 0 || n >= kMaxN || num_rows < 0 || k < 1)
        return fail(DR_ERR_INVALID_ARGUMENT, "%s: need 0 <= n < 2^31, num_rows >= 0, k >= 1", what);
    if (row_bytes < 16 || row_bytes % 16 != 0)
        return fail(DR_ERR_INVALID_ARGUMENT, "%s: row_bytes must be a positive multiple of 16", what);
    if (n > 0 && (!rows || !perm || !out)) return fail(DR_ERR_INVALID_ARGUMENT, "%s: null pointer", what);
    if (n > 0 && (!aligned(rows, 16) || !aligned(out, 16) || !aligned(perm, 4) || !aligned(inv_perm, 4)))
        return fail(DR_ERR_INVALID_ARGUMENT, "%s: rows and out must be 16-byte aligned", what);
    if (dev_status && !aligned(dev_status, 4)) return fail(DR_ERR_INVALID_ARGUMENT, "%s: misaligned dev_status", what);
    DR_TRY_HIP(dr::launch_permute_rows(rows, row_bytes, num_rows, perm, inv_perm, n, k, out, dev_status, stream),
               "permute launch");
    return ok();
}

// ---------------------------------------------------------------------------
namespace {
constexpr int64_t kDecodeDim = 128;
constexpr int32_t kMaxDecodeLen = 1 << 30;
constexpr int32_t kMaxKvChunk = 1 << 20;

bool decode_shape_ok(int64_t batch, int32_t hq, int32_t hkv, int64_t head_dim, int32_t max_seq_len, int32_t kv_chunk) {
    if (batch < 0 || hq < 1 || hkv < 1 || head_dim != kDecodeDim) return false;
    if (max_seq_len < 1 || max_seq_len > kMaxDecodeLen) return false;
    if (kv_chunk < 64 || kv_chunk > kMaxKvChunk || kv_chunk % 64 != 0) return false;
    if (hq % hkv != 0) return false;
    const int32_t g = hq / hkv;
    if (g != 1 && g != 2 && g != 4 && g != 8 && g != 16) return false;
    const int64_t nc = dr::decode_num_chunks(max_seq_len, kv_chunk);
    if (batch > 0 && (batch * hkv >= kMaxN || batch * hkv * nc >= kMaxN || batch * hq >= kMaxN)) return false;
    return true;
}

size_t decode_slots_bytes(int64_t batch, int32_t hq, int32_t max_seq_len, int32_t kv_chunk) {
    const int64_t slots = batch * hq * dr::decode_num_chunks(max_seq_len, kv_chunk);
    return (size_t)slots * (sizeof(float2) + kDecodeDim * sizeof(float));
}
}  // namespace

size_t dr_decode_attention_workspace_size(int64_t batch, int32_t num_q_heads, int32_t max_seq_len, int32_t kv_chunk,
                                          int64_t head_dim) {
    if (batch < 0 || num_q_heads < 1 || head_dim != kDecodeDim || max_seq_len < 1 || max_seq_len > kMaxDecodeLen ||
        kv_chunk < 64 || kv_chunk > kMaxKvChunk || kv_chunk % 64 != 0)
        return 0;
    return dr::kStatusBytes + decode_slots_bytes(batch, num_q_heads, max_seq_len, kv_chunk);
}

dr_status dr_decode_attention(float* out, const void* q, const void* k_cache, const void* v_cache,
                              dr_kv_layout kv_layout, const int32_t* seq_lens, int64_t batch, int32_t num_q_heads,
                              int32_t num_kv_heads, int64_t head_dim, int32_t max_seq_len, float scale,
                              int32_t kv_chunk, void* ws, size_t ws_bytes, int32_t* dev_status, hipStream_t stream) {
    const char* what = "dr_decode_attention";
    if (kv_layout != DR_KV_TOKEN_MAJOR && kv_layout != DR_KV_HEAD_MAJOR)
        return fail(DR_ERR_INVALID_ARGUMENT, "%s: unknown KV cache layout %d", what, (int)kv_layout);
    if (!decode_shape_ok(batch, num_q_heads, num_kv_heads, head_dim, max_seq_len, kv_chunk))
        return fail(DR_ERR_INVALID_ARGUMENT,
                    "%s: need head_dim 128, num_q_heads / num_kv_heads in {1, 2, 4, 8, 16}, "
                    "1 <= max_seq_len <= 2^30, kv_chunk a multiple of 64 in [64, 2^20], and fewer than 2^31 "
                    "workgroups",
                    what);
    if (!(scale == scale) || scale == __builtin_inff() || scale == -__builtin_inff())
        return fail(DR_ERR_INVALID_ARGUMENT, "%s: scale must be finite", what);
    if (batch == 0) return ok();
    if (!out || !q || !k_cache || !v_cache || !seq_lens || !ws)
        return fail(DR_ERR_INVALID_ARGUMENT, "%s: null pointer", what);
    if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
        !aligned(seq_lens, 4) || !aligned(ws, 16) || (dev_status && !aligned(dev_status, 4)))
        return fail(DR_ERR_INVALID_ARGUMENT, "%s: misaligned pointer", what);
    const size_t need = dr_decode_attention_workspace_size(batch, num_q_heads, max_seq_len, kv_chunk, head_dim);
    if (ws_bytes < need)
        return fail(DR_ERR_WORKSPACE_TOO_SMALL, "%s: workspace has %zu bytes, needs %zu", what, ws_bytes, need);
    char* base = static_cast<char*>(ws) + dr::kStatusBytes;
    const int64_t slots = batch * num_q_heads * dr::decode_num_chunks(max_seq_len, kv_chunk);
    float2* ml = reinterpret_cast<float2*>(base);
    float* po = reinterpret_cast<float*>(base + (size_t)slots * sizeof(float2));
    DR_TRY_HIP(dr::launch_decode_attention(out, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_cache),
                                           static_cast<const uint16_t*>(v_cache), seq_lens, batch, num_q_heads,
                                           num_kv_heads, max_seq_len, kv_layout == DR_KV_HEAD_MAJOR, scale, kv_chunk,
                                           ml, po, dev_status, stream),
               "decode attention launch");
    return ok();
}

int32_t dr_decode_attention_occupancy_chunk(int64_t batch, int32_t num_kv_heads, int32_t max_seq_len) {
    if (batch < 1 || num_kv_heads < 1 || max_seq_len < 1 || max_seq_len > kMaxDecodeLen) return 0;
    const int64_t want = 2 * (int64_t)dr::device_cu_count();  // workgroups to fill the device twice over
    const int64_t per_chunk = batch * num_kv_heads;            // workgroups per chunk index
    int64_t splits = (want + per_chunk - 1) / per_chunk;
    if (splits < 1) splits = 1;
    int64_t chunk = ((max_seq_len + splits - 1) / splits + 63) / 64 * 64;
    if (chunk < 64) chunk = 64;
    if (chunk > kMaxKvChunk) chunk = kMaxKvChunk;
    return (int32_t)chunk;
}

// ---------------------------------------------------------------------------
size_t dr_fingerprint_workspace_size(int64_t nbytes) {
    (void)nbytes;
    return dr::kStatusBytes + dr::kMaxFingerprintBlocks * sizeof(uint64_t);
}

dr_status dr_fingerprint(const void* data, int64_t nbytes, uint64_t* out_hash, void* ws, size_t ws_bytes,
                         hipStream_t stream) {
    const char* what = "dr_fingerprint";
    if (nbytes < 0) return fail(DR_ERR_INVALID_ARGUMENT, "%s: nbytes must be >= 0", what);
    if (nbytes > 0 && (!data || !aligned(data, 8)))
        return fail(DR_ERR_INVALID_ARGUMENT, "%s: data must be non-null and 8-byte aligned", what);
    if (!out_hash || !aligned(out_hash, 8)) return fail(DR_ERR_INVALID_ARGUMENT, "%s: bad out_hash", what);
    if (!ws || !aligned(ws, 16)) return fail(DR_ERR_INVALID_ARGUMENT, "%s: bad workspace", what);
    if (ws_bytes < dr_fingerprint_workspace_size(nbytes))
        return fail(DR_ERR_WORKSPACE_TOO_SMALL, "%s: workspace has %zu bytes, needs %zu", what, ws_bytes,
                    dr_fingerprint_workspace_size(nbytes));
    uint64_t* partials = reinterpret_cast<uint64_t*>(static_cast<char*>(ws) + dr::kStatusBytes);
    DR_TRY_HIP(dr::launch_fingerprint(data, nbytes, out_hash, partials, stream), "fingerprint launch");
    return ok();
}

// ---------------------------------------------------------------------------
dr_status dr_read_status(const int32_t* dev_status, hipStream_t stream) {
    if (!dev_status) return fail(DR_ERR_INVALID_ARGUMENT, "dr_read_status: null pointer");
    int32_t v = 0;
    DR_TRY_HIP(hipMemcpyAsync(&v, dev_status, sizeof v, hipMemcpyDeviceToHost, stream), "status copy");
    DR_TRY_HIP(hipStreamSynchronize(stream), "stream synchronize");
    if (v == 0) return ok();
    if (v & dr::kStatusPlan) return fail(DR_ERR_BAD_PLAN, "device reported an inconsistent plan (status word %d)", v);
    return fail(DR_ERR_INDEX_OUT_OF_RANGE, "device reported an index out of range (status word %d)", v);
}

dr_status dr_workspace_status(const void* ws, hipStream_t stream) {
    if (!ws) return fail(DR_ERR_INVALID_ARGUMENT, "dr_workspace_status: null workspace");
    return dr_read_status(static_cast<const int32_t*>(ws), stream);
}

}  // extern "C"
