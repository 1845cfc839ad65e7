// Grouped-GEMM weight gradient with private token slots, merged in slot order,
// for expert shapes (large M and N).
//
// dW[g] = X_g^T dY_g for every group (expert) g, where group g owns the
// expert-major tokens [off[g], off[g+1]).  The group's tokens are cut into
// private slots of `split` tokens from its first token (the last one short);
// slot s's partial P_s = X_s^T dY_s is accumulated in token order with the
// bf16 MFMA into fp32, and dW[g] = T(P_0, ..., P_{S_g-1}): chunks of 8 slots
// summed left to right, the chunk sums combined by the pairwise tree.  This is
// the private-slot fix the pages give for the grouped-GEMM epilogue (every
// writer gets its own slot, merged in a fixed order: bitwise-determinism
// interview note, "where nondeterminism comes from", multiple-writers row;
// Megatron-LM determinism reference, section 3.3, grouped-GEMM wgrad).  The
// bits equal those of dr_grouped_splitk_gemm_tn + dr_grouped_splitk_reduce:
// the same MFMA sequence per slot and the same tree.
//
// Where the thin split-K kernel streams X once past 32-column tiles, here a
// workgroup owns a 256 (M) x 128 (N) output tile of one chunk of one group and
// walks the chunk's slots: each slot's partial is accumulated in registers
// (8 wavefronts, a 4 x 2 grid of 64 x 64 blocks), then added into the chunk's
// running sum, also in registers, so the partials never go to memory.  The
// two sets take 128 registers per lane, so two wavefronts fit on each SIMD
// and one's waits are covered by the other's MFMAs (with 64 x 128 blocks the
// sets took 256 registers and one wavefront per SIMD ran about 1.25 times slower,
// although it reads less from LDS per MFMA).  A group of at most 8 slots
// writes dW[g] directly; a longer group writes its chunk sums to a workspace,
// and a merge kernel applies the pairwise tree over them in chunk order.
//
// Stages of 64 tokens go from global memory straight into LDS (16-byte
// direct loads, gfx950), in their natural token-major layout, into a ring of
// three stage buffers: the loads of stage j+2 fly while stage j is computed.
// The loads go through a buffer resource over the stage's token rows, so rows
// past a slot's end and columns past the matrix read zeros from the range
// check and each lane's offset is fixed for a tile; the stage's base address
// is the only per-stage work of the load side.  The MFMA operands (8
// consecutive tokens of one column) come out of LDS with the transposing read
// ds_read_b64_tr_b16 (two per operand): lane j of a 16-lane group receives
// column j of the group's 4-token x 16-column block, and the next k-step's
// reads are issued before the current k-step's MFMAs.  The 16-byte chunks of
// a row are XOR-swizzled by the row's low two bits, so the four rows a
// transposing read touches fall in different banks.
#include "internal.h"
#include "lds_tile.h"

namespace dr {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int TM = 256;          // output rows (M) per workgroup
constexpr int TN = 128;          // output columns (N) per workgroup
constexpr int TK = 64;           // tokens per stage
constexpr int kThreads = 512;    // 8 wavefronts, each 64 (M) x 64 (N)
constexpr int kChunk = 8;        // slots summed left to right before the pairwise tree

struct Plan {
    const int32_t* cum_items;   // [G + 1] work items before each group
    const int32_t* chunk_base;  // [G] first chunk-sum row of a group of more than one chunk, else -1
};

// One work item: chunk c of group g, output tile (m0, n0).
struct Item {
    int32_t g, c;
    int64_t m0, n0;
    int32_t t0, t1;     // the group's tokens
    int32_t slot0;      // first slot of the chunk
    int32_t nslots;     // slots of the chunk (0 for an empty group)
    float* dst;         // dW[g] or the chunk's sum row
};

__device__ __forceinline__ Item item_of(uint32_t it, const int32_t* __restrict__ off, int32_t G, int32_t split,
                                        uint32_t mtiles, uint32_t ntiles, int64_t M, int64_t N, const Plan& p,
                                        float* __restrict__ out, float* __restrict__ chunks) {
    // the group: the last g with cum_items[g] <= it
    int32_t lo = 0, hi = G;  // invariant: cum_items[lo] <= it < cum_items[hi]
    while (hi - lo > 1) {
        const int32_t mid = (lo + hi) >> 1;
        if ((uint32_t)p.cum_items[mid] <= it) lo = mid;
        else hi = mid;
    }
    Item w;
    w.g = lo;
    const uint32_t local = it - (uint32_t)p.cum_items[lo];
    const uint32_t tiles = mtiles * ntiles;
    w.c = (int32_t)(local / tiles);
    // tiles in bands of 8 N tiles, each band M row by M row: 32 consecutive
    // tiles are 4 M panels x 8 N tiles
    const uint32_t t = local - (uint32_t)w.c * tiles;
    const uint32_t band = t / (mtiles * 8u), u = t - band * (mtiles * 8u);
    const uint32_t wb = min(8u, ntiles - band * 8u);
    w.m0 = (int64_t)(u / wb) * TM;
    w.n0 = (int64_t)(band * 8u + u % wb) * TN;
    w.t0 = off[lo];
    w.t1 = off[lo + 1];
    const int32_t slots = (int32_t)(((uint32_t)(w.t1 - w.t0) + (uint32_t)split - 1u) / (uint32_t)split);
    w.slot0 = w.c * kChunk;
    w.nslots = min(kChunk, slots - w.slot0);
    if (w.nslots < 0) w.nslots = 0;
    const int32_t cb = p.chunk_base[lo];
    w.dst = cb < 0 ? out + (int64_t)lo * M * N : chunks + (int64_t)(cb + w.c) * M * N;
    return w;
}

// The walk of one worker over its stages: item by item (items w, w + P, ...),
// within an item the chunk's slots in order, within a slot 64-token stages
// from its first token (the last one short).  An empty group's item is one
// stage of no tokens.  All fields are wave-uniform.
struct Cursor {
    uint32_t it;        // current item
    int32_t t;          // the stage's first token
    int32_t te;         // end of the stage's slot
    int32_t ce;         // end of the item's chunk
    int64_t m0, n0;     // the item's tile
    int32_t valid;      // flag: a stage of this worker (0 past its last)
};

__device__ __forceinline__ void cursor_item(Cursor& c, uint32_t it, uint32_t items, const int32_t* __restrict__ off,
                                            int32_t G, int32_t split, uint32_t mtiles, uint32_t ntiles, int64_t M,
                                            int64_t N, const Plan& plan, float* __restrict__ out,
                                            float* __restrict__ chunks) {
    c.it = it;
    c.valid = it < items;
    if (!c.valid) return;
    const Item w = item_of(it, off, G, split, mtiles, ntiles, M, N, plan, out, chunks);
    const int64_t cs = (int64_t)w.t0 + (int64_t)w.slot0 * split;
    c.t = w.nslots ? (int32_t)cs : w.t0;
    c.ce = w.nslots ? (int32_t)min((int64_t)w.t1, cs + (int64_t)w.nslots * split) : w.t0;
    c.te = (int32_t)min((int64_t)c.ce, (int64_t)c.t + split);
    c.m0 = w.m0;
    c.n0 = w.n0;
}

// The stage's descriptor for the compute side: token rows (0..64) in bits
// 0..7, slot-last in bit 8, chunk-last in bit 9.
__device__ __forceinline__ uint32_t cursor_desc(const Cursor& c) {
    const int32_t rows = max(0, min(TK, c.te - c.t));
    const uint32_t slot_last = c.t + TK >= c.te;
    const uint32_t chunk_last = slot_last && c.te >= c.ce;
    return (uint32_t)rows | slot_last << 8 | chunk_last << 9;
}

// The stages of an item: ceil(tokens / TK) per slot of its chunk, one for an
// empty group (the walk of the kernel's load cursor).
__device__ __forceinline__ uint32_t item_stages(const Item& w, int32_t split) {
    if (w.nslots == 0) return 1u;
    const int64_t cs = (int64_t)w.t0 + (int64_t)w.slot0 * split;
    const int64_t last = min((int64_t)w.t1, cs + (int64_t)w.nslots * split) - (cs + (int64_t)(w.nslots - 1) * split);
    return (uint32_t)(w.nslots - 1) * (uint32_t)((split + TK - 1) / TK) + (uint32_t)((last + TK - 1) / TK);
}

constexpr uint32_t kOutOfRange = 0x80000000u;  // a byte offset past every buffer range
constexpr int kXLoads = TM * TK * 2 / 16 / kThreads;  // 16-byte direct loads per thread per stage: 8
constexpr int kYLoads = TN * TK * 2 / 16 / kThreads;  // 4

// Byte offset of this thread's direct-load piece k of a stage, from the
// stage's first token row at the tile's first column: instruction k of
// wavefront w fills the 1 KB at position 64 (n w + k) of the LDS tile (lane L
// at 16 L, n the instructions per thread), position p being token row
// p / (COLS / 8) and 16-byte chunk p % (COLS / 8), swizzled as in lds_at.
// A chunk whose columns are past the matrix gets an offset past every range.
template <int COLS>
__device__ __forceinline__ uint32_t piece_offset(int k, int64_t ld, int64_t col0, int64_t cols_total) {
    constexpr int kChunks = COLS / 8;
    constexpr int kLoads = COLS * TK * 2 / 16 / kThreads;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int pos = 64 * (kLoads * wv + k) + lane;
    const int r = pos / kChunks;
    const int cc = (pos % kChunks) ^ ((r & 3) << 2);
    return col0 + 8 * cc < cols_total ? (uint32_t)(r * ld * 2 + 16 * cc) : kOutOfRange;
}

// The direct loads of one stage of a token-major matrix into an LDS tile,
// through a buffer resource over the stage's rows: its range check returns
// zeros for the token rows at or past `rows` and for the out-of-range offset.
template <int COLS>
__device__ __forceinline__ void dma_stage(const uint16_t* base, int64_t ld, int32_t rows, const uint32_t* voff,
                                          uint16_t* tile) {
    constexpr int kLoads = COLS * TK * 2 / 16 / kThreads;
    const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    // the stage's base and size are wave-uniform: say so, so that the
    // resource is built in scalar registers once
    const uint64_t bp = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)bp);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(bp >> 32));
    const int nbytes = __builtin_amdgcn_readfirstlane((int)(rows * ld * 2));
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<uint16_t*>((uint64_t)hi << 32 | lo), 0, nbytes, 0x00020000);
#pragma unroll
    for (int k = 0; k < kLoads; ++k)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(tile + 64 * (kLoads * wv + k) * 8), 16, voff[k], 0,
                                                 0, 0);
}

typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
struct KRaw {
    u32x2v r[8];
};

// Issues the eight transposing reads of k-step ks; their registers are not
// valid until wait_kstep.  The compiler does not see them as LDS reads (so it
// adds no wait on the direct loads in flight for later stages); wait_kstep
// takes the registers as operands, so no use of them moves above the wait.
__device__ __forceinline__ void issue_kstep(KRaw& k, const uint16_t* xt, const uint16_t* yt, const int (&xoff)[2],
                                            const int (&yoff)[2], int ks) {
    const uint32_t xb = lds_byte_address(xt, 16 * ks * TM), yb = lds_byte_address(yt, 16 * ks * TN);
    const uint32_t a0 = xb + 2 * xoff[0], a1 = xb + 2 * xoff[1];
    const uint32_t b0 = yb + 2 * yoff[0], b1 = yb + 2 * yoff[1];
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8\n"
        "ds_read_b64_tr_b16 %1, %8 offset:2048\n"
        "ds_read_b64_tr_b16 %2, %9\n"
        "ds_read_b64_tr_b16 %3, %9 offset:2048\n"
        "ds_read_b64_tr_b16 %4, %10\n"
        "ds_read_b64_tr_b16 %5, %10 offset:1024\n"
        "ds_read_b64_tr_b16 %6, %11\n"
        "ds_read_b64_tr_b16 %7, %11 offset:1024"
        : "=&v"(k.r[0]), "=&v"(k.r[1]), "=&v"(k.r[2]), "=&v"(k.r[3]), "=&v"(k.r[4]), "=&v"(k.r[5]), "=&v"(k.r[6]),
          "=&v"(k.r[7])
        : "v"(a0), "v"(a1), "v"(b0), "v"(b1)
        : "memory");
}

__device__ __forceinline__ void wait_kstep(KRaw& k) {
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(k.r[0]), "+v"(k.r[1]), "+v"(k.r[2]), "+v"(k.r[3]), "+v"(k.r[4]), "+v"(k.r[5]), "+v"(k.r[6]),
                   "+v"(k.r[7])
                 :
                 : "memory");
}

__device__ __forceinline__ void mfma_kstep(f32x16 (&acc)[2][2], const KRaw& k) {
    typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
    bf16x8 a[2], b[2];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const u32x4v v{k.r[2 * q][0], k.r[2 * q][1], k.r[2 * q + 1][0], k.r[2 * q + 1][1]};
        if (q < 2) a[q] = __builtin_bit_cast(bf16x8, v);
        else b[q - 2] = __builtin_bit_cast(bf16x8, v);
    }
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mb], b[nb], acc[mb][nb], 0, 0, 0);
}

// The chunk sum s (or the empty group's zero tile) to its destination.  In
// wavefront (wm, wn), lane (i, h) holds column 64 wn + 32 nb + i and rows
// 64 wm + 32 mb + 8 (v/4) + 4h + v%4 of the tile.
// One 32x32 block at a time, walking one row pointer, so that few addresses
// are live at once.
__device__ __forceinline__ void store_tile(const f32x16 (&s)[2][2], float* dst, int64_t m0, int64_t n0, int64_t M,
                                           int64_t N) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int wm = wv & 3, wn = wv >> 2;
    const int i = lane & 31, h = lane >> 5;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            const int64_t m_first = m0 + 64 * wm + 32 * mb + 4 * h;
            const int64_t n = n0 + 64 * wn + 32 * nb + i;
            float* p = dst + m_first * N + n;
            const bool col_ok = n < N;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int dm = 8 * (v / 4) + (v % 4);
                if (col_ok && m_first + dm < M) __builtin_nontemporal_store(s[mb][nb][v], p);
                p += (v % 4 == 3) ? 5 * N : N;
            }
            __builtin_amdgcn_sched_barrier(0);
        }
}

// Persistent workgroups; worker w takes items w, w + P, w + 2P, ...  Logical
// workers are numbered XCD by XCD (workgroup b runs on XCD b mod 8), so the
// 32 items in flight at one time on one XCD are 4 M panels x 8 N tiles of one
// group: each X stage is read by 8 of them and each dY stage by 4, mostly
// from that XCD's L2.
//
// Stages go through a ring of three LDS buffers: the direct loads of stage
// j + 2 are issued while stage j is computed.  The load side walks a cursor
// two stages ahead of the compute side, which sees each stage as a
// descriptor (rows and slot and chunk ends) and the item it belongs to.
__global__ __launch_bounds__(kThreads, 1) void wgrad_kernel(const uint16_t* __restrict__ X,
                                                            const uint16_t* __restrict__ dY, int64_t K, int64_t M,
                                                            int64_t N, const int32_t* __restrict__ off, int32_t G,
                                                            int32_t split, uint32_t mtiles, uint32_t ntiles,
                                                            const int32_t* __restrict__ cum_items,
                                                            const int32_t* __restrict__ chunk_base,
                                                            const int32_t* __restrict__ status,
                                                            float* __restrict__ out, float* __restrict__ chunks) {
    __shared__ __attribute__((aligned(1024))) uint16_t xs[3][TM * TK];
    __shared__ __attribute__((aligned(1024))) uint16_t ys[3][TN * TK];
    if (status[kWordStatus] != 0) return;  // the offsets failed the plan's check: nothing is written
    const Plan plan{cum_items, chunk_base};
    const uint32_t items = (uint32_t)plan.cum_items[G];
    const uint32_t P = gridDim.x;
    const uint32_t b = blockIdx.x;
    const uint32_t wkr = (P % 8 == 0) ? (b % 8) * (P / 8) + b / 8 : b;
    if (wkr >= items) return;
    const int wv = threadIdx.x >> 6;
    int xoff[2], yoff[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) xoff[mb] = operand_offset<TM>(64 * (wv & 3) + 32 * mb);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) yoff[nb] = operand_offset<TN>(64 * (wv >> 2) + 32 * nb);

    // The load side: its cursor and the piece offsets of its item's tile.
    Cursor ld;
    uint32_t xv[kXLoads], yv[kYLoads];
    auto tile_offsets = [&]() {
#pragma unroll
        for (int k = 0; k < kXLoads; ++k) xv[k] = piece_offset<TM>(k, M, ld.m0, M);
#pragma unroll
        for (int k = 0; k < kYLoads; ++k) yv[k] = piece_offset<TN>(k, N, ld.n0, N);
    };
    cursor_item(ld, wkr, items, off, G, split, mtiles, ntiles, M, N, plan, out, chunks);
    tile_offsets();
    // Every call issues the same loads (a stage past the worker's last has no
    // rows and reads zeros), so each stage adds the same count to the vector
    // memory counter.
    auto issue = [&](uint16_t* xt, uint16_t* yt) {
        const int32_t rows = ld.valid ? max(0, min(TK, ld.te - ld.t)) : 0;
        const int64_t t = ld.valid ? ld.t : 0, m0 = ld.valid ? ld.m0 : 0, n0 = ld.valid ? ld.n0 : 0;
        dma_stage<TM>(X + t * M + m0, M, rows, xv, xt);
        dma_stage<TN>(dY + t * N + n0, N, rows, yv, yt);
    };
    auto advance = [&]() {
        if (!ld.valid) return;
        if (ld.t + TK < ld.te) {
            ld.t += TK;
        } else if (ld.te < ld.ce) {
            ld.t = ld.te;
            ld.te = (int32_t)min((int64_t)ld.ce, (int64_t)ld.te + split);
        } else {
            cursor_item(ld, ld.it + P, items, off, G, split, mtiles, ntiles, M, N, plan, out, chunks);
            if (ld.valid) tile_offsets();
        }
    };

    // the worker's stage count, so that the loop below has no exit inside its three steps
    uint32_t stages = 0;
    for (uint32_t it = wkr; it < items; it += P)
        stages += item_stages(item_of(it, off, G, split, mtiles, ntiles, M, N, plan, out, chunks), split);

    f32x16 acc[2][2], sum[2][2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                acc[mb][nb][v] = 0.f;
                sum[mb][nb][v] = neg_zero();
            }

    // the compute side's view of the two stages in flight
    uint32_t d_cur = cursor_desc(ld), it_cur = ld.it;
    issue(xs[0], ys[0]);
    advance();
    uint32_t d_nx1 = cursor_desc(ld), it_nx1 = ld.it;
    issue(xs[1], ys[1]);
    advance();

    auto step = [&](const uint16_t* xt, const uint16_t* yt, uint16_t* xn, uint16_t* yn) {
        // This stage's pieces have landed once at most the next stage's are
        // outstanding; after the barrier every wavefront's have, and every
        // wavefront is done reading xn / yn (the previous stage's buffers,
        // whose operands its MFMAs consumed).  A plain barrier: the workgroup
        // fences of __syncthreads would wait for the loads still in flight.
        DR_WAIT_VMCNT(kXLoads + kYLoads);
        __builtin_amdgcn_s_barrier();
        const uint32_t d_nx2 = cursor_desc(ld), it_nx2 = ld.it;
        issue(xn, yn);
        advance();
        const int ksteps = (int)((d_cur & 0xFFu) + 15) >> 4;
        if (ksteps > 0) {
            KRaw kr[2];
            issue_kstep(kr[0], xt, yt, xoff, yoff, 0);
            wait_kstep(kr[0]);
#pragma unroll
            for (int ks = 0; ks < TK / 16; ++ks) {
                if (ks >= ksteps) break;
                const bool more = ks + 1 < TK / 16 && ks + 1 < ksteps;
                // the next k-step's reads run while these MFMAs execute
                if (more) issue_kstep(kr[(ks + 1) & 1], xt, yt, xoff, yoff, ks + 1);
                __builtin_amdgcn_sched_barrier(0);
                mfma_kstep(acc, kr[ks & 1]);
                __builtin_amdgcn_sched_barrier(0);
                if (more) wait_kstep(kr[(ks + 1) & 1]);
            }
        }
        if (d_cur & 0x100u) {
            // the slot's partial joins the chunk's left-to-right sum, which
            // starts as -0.0 (an exact additive identity: -0.0 + x is x for
            // every x, -0.0 included), so the first slot's partial enters
            // unchanged
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        sum[mb][nb][v] = sum[mb][nb][v] + acc[mb][nb][v];
                        acc[mb][nb][v] = 0.f;
                    }
                    // one 16-value block at a time: keeps the copies out of the accumulators few
                    __builtin_amdgcn_sched_barrier(0);
                }
            if (d_cur & 0x200u) {
                const Item w = item_of(it_cur, off, G, split, mtiles, ntiles, M, N, plan, out, chunks);
                store_tile(sum, w.dst, w.m0, w.n0, M, N);
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                        for (int v = 0; v < 16; ++v) sum[mb][nb][v] = neg_zero();
            }
        }
        d_cur = d_nx1;
        it_cur = it_nx1;
        d_nx1 = d_nx2;
        it_nx1 = it_nx2;
    };
    uint32_t j = 0;
    for (; j + 3 <= stages; j += 3) {
        step(xs[0], ys[0], xs[2], ys[2]);
        step(xs[1], ys[1], xs[0], ys[0]);
        step(xs[2], ys[2], xs[1], ys[1]);
    }
    if (j < stages) step(xs[0], ys[0], xs[2], ys[2]);
    if (j + 1 < stages) step(xs[1], ys[1], xs[0], ys[0]);
}

// out[g] = the pairwise tree over the group's chunk sums, in chunk order
// (groups of more than one chunk; blockIdx.y = group).  Binary counter: a new
// chunk sum merges with the stored ones while the count's low bits carry, and
// the stored ones fold from the right at the end, which is the tree that
// splits at the largest power of two below the chunk count.
constexpr int kMergeThreads = 256;
constexpr int kMergeDepth = 24;
__global__ __launch_bounds__(kMergeThreads) void wgrad_merge_kernel(const float* __restrict__ chunks,
                                                                    const int32_t* __restrict__ off,
                                                                    const int32_t* __restrict__ chunk_base,
                                                                    int32_t split, int64_t count,
                                                                    float* __restrict__ out,
                                                                    const int32_t* __restrict__ status) {
    if (status[kWordStatus] != 0) return;
    const int64_t g = blockIdx.y;
    const int32_t cb = chunk_base[g];
    if (cb < 0) return;
    const int64_t e0 = ((int64_t)blockIdx.x * kMergeThreads + threadIdx.x) * 4;
    if (e0 >= count) return;
    const uint32_t slots = ((uint32_t)(off[g + 1] - off[g]) + (uint32_t)split - 1u) / (uint32_t)split;
    const uint32_t nch = (slots + kChunk - 1) / kChunk;
    float level[kMergeDepth][4];
    for (uint32_t c = 0; c < nch; ++c) {
        const u32x4 raw = load16_stream(chunks + (int64_t)(cb + c) * count + e0);
        float v[4] = {__uint_as_float(raw.x), __uint_as_float(raw.y), __uint_as_float(raw.z),
                      __uint_as_float(raw.w)};
        bool carry = true;
#pragma unroll
        for (int l = 0; l < kMergeDepth; ++l) {
            if (carry) {
                if ((c >> l) & 1u) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = level[l][e] + v[e];
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) level[l][e] = v[e];
                    carry = false;
                }
            }
        }
    }
    float acc[4];
    bool have = false;
#pragma unroll
    for (int l = 0; l < kMergeDepth; ++l) {
        if ((nch >> l) & 1u) {
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] = have ? level[l][e] + acc[e] : level[l][e];
            have = true;
        }
    }
    store16(out + g * count + e0, u32x4{__float_as_uint(acc[0]), __float_as_uint(acc[1]), __float_as_uint(acc[2]),
                                        __float_as_uint(acc[3])});
}

// The plan, by one workgroup: per group, its chunk count (at least one work
// item per tile, also for an empty group, which gets the zero gradient), the
// cumulative work items and, for groups of more than one chunk, the first row
// of their chunk sums.  Offsets that are not non-decreasing within [0, K], or
// chunk sums beyond the workspace bound, set the status word (nothing is then
// computed or written); otherwise the word is cleared.
constexpr int kPlanThreads = 1024;
__device__ __forceinline__ int32_t block_exclusive_scan(int32_t v, int32_t* total, int32_t* wave_tot) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    int32_t incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int32_t t = __shfl_up(incl, o, 64);
        if (lane >= o) incl += t;
    }
    if (lane == 63) wave_tot[w] = incl;
    __syncthreads();
    int32_t before = 0, all = 0;
    for (int k = 0; k < kPlanThreads / 64; ++k) {
        before += k < w ? wave_tot[k] : 0;
        all += wave_tot[k];
    }
    __syncthreads();
    *total = all;
    return before + incl - v;
}

__global__ __launch_bounds__(kPlanThreads) void wgrad_plan_kernel(const int32_t* __restrict__ off, int32_t G,
                                                                  int64_t K, int32_t split, int64_t tiles,
                                                                  int64_t max_items, int64_t max_chunk_rows,
                                                                  int32_t* __restrict__ cum_items,
                                                                  int32_t* __restrict__ chunk_base,
                                                                  int32_t* __restrict__ status) {
    __shared__ int32_t wave_tot[2][kPlanThreads / 64];
    const int tid = threadIdx.x;
    int64_t item_carry = 0, chunk_carry = 0;
    int bad = 0;
    for (int32_t g0 = 0; g0 < G; g0 += kPlanThreads) {
        const int32_t g = g0 + tid;
        int32_t nitems = 0, nchunk_rows = 0;
        if (g < G) {
            const int32_t a = off[g], b = off[g + 1];
            if (a < 0 || b < a || (int64_t)b > K) {
                bad = 1;
            } else {
                const uint32_t slots = ((uint32_t)(b - a) + (uint32_t)split - 1u) / (uint32_t)split;
                const int32_t nch = (int32_t)((slots + kChunk - 1) / kChunk);
                nitems = (nch > 1 ? nch : 1) * (int32_t)tiles;  // the host bounds the total below 2^31
                nchunk_rows = nch > 1 ? nch : 0;
            }
        }
        int32_t it_total, ch_total;
        const int32_t it_before = block_exclusive_scan(nitems, &it_total, wave_tot[0]);
        const int32_t ch_before = block_exclusive_scan(nchunk_rows, &ch_total, wave_tot[1]);
        if (g < G) {
            cum_items[g] = (int32_t)min(item_carry + it_before, max_items);
            chunk_base[g] = nchunk_rows ? (int32_t)min(chunk_carry + ch_before, max_chunk_rows) : -1;
        }
        item_carry += it_total;
        chunk_carry += ch_total;
    }
    if (item_carry > max_items || chunk_carry > max_chunk_rows) bad = 1;
    bad = __syncthreads_or(bad);
    if (tid == 0) {
        cum_items[G] = bad ? 0 : (int32_t)item_carry;
        status[kWordStatus] = bad ? kStatusPlan : 0;
    }
}

}  // namespace

int64_t wgrad_max_chunk_rows(int64_t K, int32_t split) {
    // a group of C >= 2 chunks has C <= 2 (C - 1) and C - 1 <= (K_g - 1) / (8 split)
    return K / (4 * (int64_t)split) + 1;
}

int64_t wgrad_max_items(int64_t K, int32_t num_groups, int32_t split, int64_t M, int64_t N) {
    const int64_t tiles = ((M + TM - 1) / TM) * ((N + TN - 1) / TN);
    // sum_g max(1, C_g) <= G + K / (8 split)
    return (num_groups + K / (kChunk * (int64_t)split) + 1) * tiles;
}

hipError_t launch_wgrad(const uint16_t* X, const uint16_t* dY, int64_t K, int64_t M, int64_t N,
                        const int32_t* group_offsets, int32_t num_groups, int32_t split, float* out,
                        int32_t* status, int32_t* cum_items, int32_t* chunk_base, float* chunks, hipStream_t s) {
    const int64_t mtiles = (M + TM - 1) / TM, ntiles = (N + TN - 1) / TN;
    const int64_t max_items = wgrad_max_items(K, num_groups, split, M, N);
    hipLaunchKernelGGL(wgrad_plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, group_offsets, num_groups, K, split,
                       mtiles * ntiles, max_items, wgrad_max_chunk_rows(K, split), cum_items, chunk_base, status);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const Launch lc = launch_config();
    int64_t grid = lc.grid_blocks > 0 ? lc.grid_blocks : (int64_t)device_cu_count();
    if (grid > max_items) grid = max_items;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(wgrad_kernel, dim3((unsigned)grid), dim3(kThreads), 0, s, X, dY, K, M, N, group_offsets,
                       num_groups, split, (uint32_t)mtiles, (uint32_t)ntiles, cum_items, chunk_base, status,
                       out, chunks);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t count = M * N;
    const dim3 mgrid((unsigned)((count / 4 + kMergeThreads - 1) / kMergeThreads), (unsigned)num_groups);
    hipLaunchKernelGGL(wgrad_merge_kernel, mgrid, dim3(kMergeThreads), 0, s, chunks, group_offsets, chunk_base, split,
                       count, out, status);
    return hipGetLastError();
}

}  // namespace dr
