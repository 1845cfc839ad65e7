// Split-K thin contraction dW = X^T dY into private per-split buffers, and the
// ordered reduce over split ids.
//
// The DeepSeek-V4 mHC backward (ch. 9, section 3.3) has an output dimension of
// only 24.  It must split the contraction, and it keeps one buffer per split,
// reduced afterwards by a dedicated kernel in split-id order.  Here:
//   splitk_gemm: persistent workgroups walk contiguous ranges of (split,
//     32-column N tile, 64-row M tile) items in stages of up to 256 tokens (16
//     independent 16-byte loads per thread), staged in LDS (X row-major, dY
//     transposed, dY kept while consecutive items share it); the next stage's
//     loads are in flight while the current one is computed.  Each of the two
//     wavefronts accumulates a 32x32 tile with the bf16 MFMA
//     v_mfma_f32_32x32x16_bf16, in token order, into fp32, and the tile leaves
//     through LDS as contiguous 16-byte stores.  A partial depends only on
//     (split, m, n): not on the grid, the M/N tiling or other columns.  The HBM
//     stream is X (read once) plus the partials (written once); the MFMA work
//     is small beside it.
//   splitk_stream: the same partials for thin N (at most 32 columns, a
//     multiple of 8; the mHC shape), one persistent workgroup of eight
//     wavefronts per CU, 256-column M tiles in 64-token stages, loads two
//     stages ahead through registers; the default for those shapes (same bits).
//   splitk_reduce: out[e] = T(P_0[e], ..., P_{S-1}[e]); chunks of 8 splits left
//     to right, then the pairwise tree: for 9..512 splits a lane per chunk and
//     the tree across lanes (shuffles), else one thread per 4 consecutive
//     elements walking the chunks.
// The atomic baseline runs the same tile code and adds each split's tile into
// out with hardware fp32 atomics.
#include "internal.h"
#include "lds_tile.h"

namespace dr {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 64;   // M rows per workgroup (two 32-row wavefront tiles)
constexpr int BN = 32;   // N columns per workgroup
constexpr int KT = 256;  // tokens per LDS stage (one whole split at the mHC shape)
constexpr int kGemmThreads = 128;
// LDS row strides in bf16, multiples of 8 (16-byte aligned rows).  X is kept
// row-major [token][m]; dY is kept transposed [n][token] so that a lane's 8
// consecutive tokens of one column are one 16-byte read.
constexpr int XS = BM + 8;
constexpr int YS = KT + 8;

__device__ __forceinline__ __bf16 as_bf16(uint16_t b) { return __builtin_bit_cast(__bf16, b); }

constexpr int kLoadsPerThread = KT * (BM / 8) / kGemmThreads;  // 16-byte X loads per thread per stage

// Coordinates of one unit of work: a KT-token stage of one (split, N tile, M tile) item.
struct Unit {
    uint32_t item;  // (split, N tile, M tile), M tile fastest
    int stage;      // KT-token stage within the split
};

struct UnitGeom {
    int s;
    int64_t m0, n0, t0;
    int rows;        // valid tokens of the stage
    bool last;       // last stage of its split
    bool x_vec;      // full-width M tile with 16-byte rows
};

// 32-bit tile arithmetic: the host keeps the item count below 2^31.  With
// ranges (a grouped split), split s covers tokens [ranges[s].x, ranges[s].y).
__device__ __forceinline__ UnitGeom geometry(const Unit& u, int64_t K, int64_t M, int64_t kc, uint32_t mtiles,
                                             uint32_t ntiles, const int2* __restrict__ ranges) {
    UnitGeom g;
    const uint32_t mt = u.item % mtiles;
    const uint32_t rest = u.item / mtiles;
    const uint32_t nt = rest % ntiles;
    g.s = (int)(rest / ntiles);
    g.m0 = (int64_t)mt * BM;
    g.n0 = (int64_t)nt * BN;
    int64_t t_begin, t_end;
    if (ranges) {
        const int2 r = ranges[g.s];
        t_begin = r.x;
        t_end = r.y;
    } else {
        t_begin = (int64_t)g.s * kc;
        t_end = min(K, t_begin + kc);
    }
    g.t0 = t_begin + (int64_t)u.stage * KT;
    g.rows = (int)min((int64_t)KT, t_end - g.t0);
    g.last = g.t0 + KT >= t_end;
    g.x_vec = (M % 8) == 0 && g.m0 + BM <= M;
    return g;
}

__device__ __forceinline__ Unit next_unit(const Unit& u, const UnitGeom& g) {
    return g.last ? Unit{u.item + 1, 0} : Unit{u.item, u.stage + 1};
}

// Issues the 16-byte X loads of a full-width unit (rows past the split read as
// zero).  Plain cached loads: for 128-byte row pieces strided by the row pitch
// they sustain more bandwidth on gfx950 than loads with the streaming hint.
__device__ __forceinline__ void load_x(const uint16_t* __restrict__ X, int64_t M, const UnitGeom& g,
                                       u32x4 (&buf)[kLoadsPerThread]) {
#pragma unroll
    for (int q = 0; q < kLoadsPerThread; ++q) {
        const int p = threadIdx.x + q * kGemmThreads;
        const int r = p / (BM / 8), c8 = (p % (BM / 8)) * 8;
        buf[q] = u32x4{0u, 0u, 0u, 0u};
        if (r < g.rows) buf[q] = *reinterpret_cast<const u32x4*>(X + (g.t0 + r) * M + g.m0 + c8);
    }
}

// Output tile staging: fp32 [BM][OS] in the X stage's LDS, so that a split's
// tile leaves as contiguous 16-byte stores.
constexpr int OS = BN + 4;
static_assert(BM * OS * 4 <= KT * XS * 2, "output tile must fit in the X stage");

// Each persistent workgroup walks a contiguous range of items (consecutive M
// tiles of one split share their dY stage, which is then staged once).  The X
// loads of the next unit are issued right after the current unit is staged in
// LDS, so they are in flight during its MFMAs and epilogue.  A partial's
// accumulation order (token order within its split) is the same for any grid.
// Grouped split (ranges != null): the splits are the private slots of a slot
// table, whose count the slot kernel left in the status block; a set status
// word means the table is invalid and nothing is computed.
template <bool ATOMIC>
__global__ __launch_bounds__(kGemmThreads) void splitk_gemm_kernel(const uint16_t* __restrict__ X,
                                                                   const uint16_t* __restrict__ dY, int64_t K,
                                                                   int64_t M, int64_t N, int64_t kc, uint32_t items,
                                                                   uint32_t mtiles, uint32_t ntiles,
                                                                   float* __restrict__ out,
                                                                   const int2* __restrict__ ranges,
                                                                   const int32_t* __restrict__ status) {
    __shared__ __attribute__((aligned(16))) uint16_t xs[KT * XS];
    __shared__ __attribute__((aligned(16))) uint16_t ys[BN * YS];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const bool y_vec = (N % 8) == 0 && (reinterpret_cast<uintptr_t>(dY) & 15) == 0;
    const bool out_vec = (N % 4) == 0 && (reinterpret_cast<uintptr_t>(out) & 15) == 0;
    if (ranges) {
        if (status[kWordStatus] != 0) return;
        items = (uint32_t)status[kWordSlots] * ntiles * mtiles;  // the host bounds this below 2^31
    }
    // 32-bit range split: the host keeps items < 2^31
    const uint32_t per = items / gridDim.x, extra = items % gridDim.x, wg = blockIdx.x;
    const uint32_t begin = wg * per + min(wg, extra), end = begin + per + (wg < extra ? 1u : 0u);
    if (begin >= end) return;
    Unit u{begin, 0};
    int64_t staged_t0 = -1, staged_n0 = -1;  // the dY stage held in ys
    UnitGeom g = geometry(u, K, M, kc, mtiles, ntiles, ranges);
    u32x4 buf[kLoadsPerThread];
    if (g.x_vec) load_x(X, M, g, buf);

    f32x16 acc;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.f;

    while (true) {
        const int ksteps = (g.rows + 15) / 16;
        const int rows16 = ksteps * 16;  // rows the MFMAs read
        // X stage -> xs; rows past the split are zero
        if (g.x_vec) {
#pragma unroll
            for (int q = 0; q < kLoadsPerThread; ++q) {
                const int p = tid + q * kGemmThreads;
                const int r = p / (BM / 8), c8 = (p % (BM / 8)) * 8;
                if (r < rows16) *reinterpret_cast<u32x4*>(xs + r * XS + c8) = buf[q];
            }
        } else {
            for (int p = tid; p < rows16 * BM; p += kGemmThreads) {
                const int r = p / BM, c = p % BM;
                const int64_t m = g.m0 + c;
                xs[r * XS + c] = (r < g.rows && m < M) ? X[(g.t0 + r) * M + m] : (uint16_t)0;
            }
        }
        // dY stage -> ys transposed; columns past N are zero
        const bool stage_y = g.t0 != staged_t0 || g.n0 != staged_n0;
        staged_t0 = g.t0;
        staged_n0 = g.n0;
        if (stage_y && y_vec) {
            const int np = (int)((min(N - g.n0, (int64_t)BN) + 7) / 8);  // 8-column pieces in this N tile
            for (int p = tid; p < rows16 * np; p += kGemmThreads) {
                const int r = p / np, c8 = (p % np) * 8;
                const u32x4 v = r < g.rows ? load16(dY + (g.t0 + r) * N + g.n0 + c8) : u32x4{0u, 0u, 0u, 0u};
                ys[(c8 + 0) * YS + r] = v.x & 0xFFFF; ys[(c8 + 1) * YS + r] = v.x >> 16;
                ys[(c8 + 2) * YS + r] = v.y & 0xFFFF; ys[(c8 + 3) * YS + r] = v.y >> 16;
                ys[(c8 + 4) * YS + r] = v.z & 0xFFFF; ys[(c8 + 5) * YS + r] = v.z >> 16;
                ys[(c8 + 6) * YS + r] = v.w & 0xFFFF; ys[(c8 + 7) * YS + r] = v.w >> 16;
            }
            for (int p = tid; p < (BN - np * 8) * (rows16 / 8); p += kGemmThreads) {
                const int c = np * 8 + p / (rows16 / 8), r8 = (p % (rows16 / 8)) * 8;
                *reinterpret_cast<u32x4*>(ys + c * YS + r8) = u32x4{0u, 0u, 0u, 0u};
            }
        } else if (stage_y) {
            for (int p = tid; p < rows16 * BN; p += kGemmThreads) {
                const int r = p / BN, c = p % BN;
                const int64_t n = g.n0 + c;
                ys[c * YS + r] = (r < g.rows && n < N) ? dY[(g.t0 + r) * N + n] : (uint16_t)0;
            }
        }
        __syncthreads();
        // the next unit's X is fetched while this one is computed
        const Unit nu = next_unit(u, g);
        const bool more = nu.item < end;
        UnitGeom ng = g;
        if (more) {
            ng = geometry(nu, K, M, kc, mtiles, ntiles, ranges);
            if (ng.x_vec) load_x(X, M, ng, buf);
        }
        const int i = lane & 31, h = lane >> 5;
        for (int ks = 0; ks < ksteps; ++ks) {
            const int kk = ks * 16 + 8 * h;
            bf16x8 a;
#pragma unroll
            for (int e = 0; e < 8; ++e) a[e] = as_bf16(xs[(kk + e) * XS + wv * 32 + i]);
            const bf16x8 b = *reinterpret_cast<const bf16x8*>(ys + i * YS + kk);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
        }
        // accumulator layout of a 32x32 MFMA tile: lane holds column (lane % 32)
        // and rows 8*(v/4) + 4*(lane/32) + (v%4) for v = 0..15
        if (ATOMIC && g.last) {
            const int64_t n = g.n0 + (lane & 31);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t m = g.m0 + wv * 32 + 8 * (v / 4) + 4 * h + (v % 4);
                if (m < M && n < N) unsafeAtomicAdd(out + m * N + n, acc[v]);
                acc[v] = 0.f;
            }
        } else if (g.last) {
            __syncthreads();  // xs is free: it now holds the output tile
            float* ot = reinterpret_cast<float*>(xs);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                ot[(wv * 32 + 8 * (v / 4) + 4 * h + (v % 4)) * OS + i] = acc[v];
                acc[v] = 0.f;
            }
            __syncthreads();
            const int rows_out = (int)min(M - g.m0, (int64_t)BM), cols = (int)min(N - g.n0, (int64_t)BN);
            float* dst = out + (int64_t)g.s * M * N + g.m0 * N + g.n0;
            if (out_vec) {
                const int q4 = cols / 4;
                for (int p = tid; p < rows_out * q4; p += kGemmThreads) {
                    const int r = p / q4, c = (p % q4) * 4;
                    store16_stream(dst + (int64_t)r * N + c, *reinterpret_cast<const u32x4*>(ot + r * OS + c));
                }
            } else {
                for (int p = tid; p < rows_out * cols; p += kGemmThreads) {
                    const int r = p / cols, c = p % cols;
                    dst[(int64_t)r * N + c] = ot[r * OS + c];
                }
            }
        }
        __syncthreads();
        if (!more) break;
        u = nu;
        g = ng;
    }
}

constexpr int kReduceThreads = 256;
constexpr int kReduceDepth = 24;  // chunk sums per element < 2^24 (splits < 2^27)

// out[e0 .. e0+VEC) = T(P_0, ..., P_{S-1}) at those elements (S >= 1).
template <int VEC>
__device__ __forceinline__ void reduce_splits(const float* __restrict__ P, int S, int64_t count, int64_t e0,
                                              float* __restrict__ out) {
    float level[kReduceDepth][VEC];
    uint32_t nchunks = 0;
    for (int c0 = 0; c0 < S; c0 += 8) {
        const int m = min(8, S - c0);
        float v[8][VEC];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (j < m) {
                if (VEC == 4) {
                    const u32x4 raw = load16(P + (int64_t)(c0 + j) * count + e0);
                    v[j][0] = __uint_as_float(raw.x);
                    v[j][VEC > 1 ? 1 : 0] = __uint_as_float(raw.y);
                    v[j][VEC > 2 ? 2 : 0] = __uint_as_float(raw.z);
                    v[j][VEC > 3 ? 3 : 0] = __uint_as_float(raw.w);
                } else {
                    v[j][0] = P[(int64_t)(c0 + j) * count + e0];
                }
            }
        }
        float s[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) s[e] = v[0][e];
#pragma unroll
        for (int j = 1; j < 8; ++j) {
            if (j < m) {
#pragma unroll
                for (int e = 0; e < VEC; ++e) s[e] = s[e] + v[j][e];
            }
        }
        // binary counter over chunk sums
        bool carry = true;
#pragma unroll
        for (int l = 0; l < kReduceDepth; ++l) {
            if (carry) {
                if ((nchunks >> l) & 1u) {
#pragma unroll
                    for (int e = 0; e < VEC; ++e) s[e] = level[l][e] + s[e];
                } else {
#pragma unroll
                    for (int e = 0; e < VEC; ++e) level[l][e] = s[e];
                    carry = false;
                }
            }
        }
        ++nchunks;
    }
    float acc[VEC];
    bool have = false;
#pragma unroll
    for (int l = 0; l < kReduceDepth; ++l) {
        if ((nchunks >> l) & 1u) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[e] = have ? level[l][e] + acc[e] : level[l][e];
            have = true;
        }
    }
    if (VEC == 4) {
        store16(out + e0, u32x4{__float_as_uint(acc[0]), __float_as_uint(acc[VEC > 1 ? 1 : 0]),
                                __float_as_uint(acc[VEC > 2 ? 2 : 0]), __float_as_uint(acc[VEC > 3 ? 3 : 0])});
    } else {
        out[e0] = acc[0];
    }
}

// With fp_part (VEC == 4 only), each workgroup also writes the fingerprint
// terms of the 16-byte pieces it stored (words e0/2 and e0/2 + 1) to
// fp_part[blockIdx.x]; the thread reads back its own store.
__device__ __forceinline__ uint64_t fp_terms_of_piece(const float* out, int64_t e0) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(out + e0);
    return fp_term(((uint64_t)v.y << 32) | v.x, e0 >> 1) + fp_term(((uint64_t)v.w << 32) | v.z, (e0 >> 1) + 1);
}

template <int VEC>
__global__ __launch_bounds__(kReduceThreads) void splitk_reduce_kernel(const float* __restrict__ P, int S,
                                                                       int64_t count, float* __restrict__ out,
                                                                       uint64_t* __restrict__ fp_part) {
    const int64_t e0 = ((int64_t)blockIdx.x * kReduceThreads + threadIdx.x) * VEC;
    if (!fp_part) {
        if (e0 < count) reduce_splits<VEC>(P, S, count, e0, out);
        return;
    }
    uint64_t h = 0;
    if (e0 < count) {
        reduce_splits<VEC>(P, S, count, e0, out);
        if (VEC == 4) h = fp_terms_of_piece(out, e0);
    }
    __shared__ uint64_t fsm[kReduceThreads / 64];
    const uint64_t b = block_sum_u64(h, fsm);
    if (threadIdx.x == 0) fp_part[blockIdx.x] = b;
}

// The same tree with L lanes per output vector (L = the chunk count rounded up
// to a power of two, at most 64): lane c sums chunk c (splits 8c .. 8c+7, left
// to right), a lane without a chunk holds -0.0, and the chunk sums are paired
// by stride doubling across the L lanes, the lower chunk as the left operand.
// With the -0.0 padding that is T over the chunk sums for any chunk count.
// All of a vector's loads are in flight at once instead of one chunk after
// another.
template <int VEC, int L>
__global__ __launch_bounds__(kReduceThreads) void splitk_reduce_lanes_kernel(const float* __restrict__ P, int S,
                                                                             int64_t count,
                                                                             float* __restrict__ out,
                                                                             uint64_t* __restrict__ fp_part) {
    const int64_t t = (int64_t)blockIdx.x * kReduceThreads + threadIdx.x;
    const int c = (int)(t % L);  // this lane's chunk
    const int64_t e0 = (t / L) * VEC;
    const bool live = e0 < count;  // whole groups of L lanes share e0
    const int m = live ? max(0, min(8, S - 8 * c)) : 0;  // splits of the chunk
    float v[8][VEC];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        if (j < m) {
            const int64_t off = (int64_t)(8 * c + j) * count + e0;
            if (VEC == 4) {
                const u32x4 raw = load16_stream(P + off);
                v[j][0] = __uint_as_float(raw.x);
                v[j][VEC > 1 ? 1 : 0] = __uint_as_float(raw.y);
                v[j][VEC > 2 ? 2 : 0] = __uint_as_float(raw.z);
                v[j][VEC > 3 ? 3 : 0] = __uint_as_float(raw.w);
            } else {
                v[j][0] = P[off];
            }
        }
    }
    float s[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) s[e] = m > 0 ? v[0][e] : neg_zero();
#pragma unroll
    for (int j = 1; j < 8; ++j) {
        if (j < m) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) s[e] = s[e] + v[j][e];
        }
    }
#pragma unroll
    for (int off = 1; off < L; off <<= 1) {
        const bool upper = (c & off) != 0;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const float o = __shfl_xor(s[e], off, 64);
            s[e] = upper ? o + s[e] : s[e] + o;
        }
    }
    if (live && c == 0) {
        if (VEC == 4) {
            store16(out + e0, u32x4{__float_as_uint(s[0]), __float_as_uint(s[VEC > 1 ? 1 : 0]),
                                    __float_as_uint(s[VEC > 2 ? 2 : 0]), __float_as_uint(s[VEC > 3 ? 3 : 0])});
        } else {
            out[e0] = s[0];
        }
    }
    if (fp_part) {
        // the fingerprint terms of the stored piece (VEC == 4 only), summed per workgroup
        uint64_t h = 0;
        if (VEC == 4 && live && c == 0) {
            const uint64_t w0 = ((uint64_t)__float_as_uint(s[VEC > 1 ? 1 : 0]) << 32) | __float_as_uint(s[0]);
            const uint64_t w1 =
                ((uint64_t)__float_as_uint(s[VEC > 3 ? 3 : 0]) << 32) | __float_as_uint(s[VEC > 2 ? 2 : 0]);
            h = fp_term(w0, e0 >> 1) + fp_term(w1, (e0 >> 1) + 1);
        }
        __shared__ uint64_t fsm[kReduceThreads / 64];
        const uint64_t b = block_sum_u64(h, fsm);
        if (threadIdx.x == 0) fp_part[blockIdx.x] = b;
    }
}

// Group g (blockIdx.y): out[g] = T over its slots slot_offsets[g] .. slot_offsets[g+1]-1,
// in slot order; a group with no slot gets the zero gradient.
template <int VEC>
__global__ __launch_bounds__(kReduceThreads) void grouped_reduce_kernel(const float* __restrict__ P,
                                                                        const int32_t* __restrict__ slot_offsets,
                                                                        int64_t max_slots, int64_t count,
                                                                        float* __restrict__ out,
                                                                        const int32_t* __restrict__ status) {
    if (status[kWordStatus] != 0) return;
    const int64_t e0 = ((int64_t)blockIdx.x * kReduceThreads + threadIdx.x) * VEC;
    if (e0 >= count) return;
    const int64_t g = blockIdx.y;
    const int32_t lo = slot_offsets[g], hi = slot_offsets[g + 1];
    if (lo < 0 || hi < lo || hi > max_slots) return;  // the slot kernel never writes such a table
    float* o = out + g * count;
    if (hi == lo) {
        if (VEC == 4) store16(o + e0, u32x4{0u, 0u, 0u, 0u});
        else o[e0] = 0.f;
        return;
    }
    reduce_splits<VEC>(P + (int64_t)lo * count, hi - lo, count, e0, o);
}

// The private slots of a grouped split, by one workgroup: group g owns tokens
// [off[g], off[g+1]), cut into consecutive slots of `split` tokens from its
// first token; slots are numbered in (group, position) order.  Writes
// slot_offsets[0 .. G], each slot's token range, and the status block (its
// word cleared, or set when the offsets are not non-decreasing within
// [0, K]; the slot count in kWordSlots).
constexpr int kSlotThreads = 1024;
__global__ __launch_bounds__(kSlotThreads) void grouped_slots_kernel(const int32_t* __restrict__ off, int32_t G,
                                                                     int64_t K, int32_t split, int64_t max_slots,
                                                                     int32_t* __restrict__ slot_offsets,
                                                                     int2* __restrict__ ranges,
                                                                     int32_t* __restrict__ status) {
    __shared__ int32_t wave_tot[kSlotThreads / 64];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    int64_t carry = 0;
    int bad = 0;
    for (int32_t g0 = 0; g0 < G; g0 += kSlotThreads) {
        const int32_t g = g0 + tid;
        int32_t a = 0, b = 0, cnt = 0;
        if (g < G) {
            a = off[g];
            b = off[g + 1];
            if (a < 0 || b < a || (int64_t)b > K) bad = 1;
            else cnt = (int32_t)(((uint32_t)(b - a) + (uint32_t)split - 1u) / (uint32_t)split);
        }
        // exclusive scan of the slot counts over the workgroup
        int32_t incl = cnt;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int32_t t = __shfl_up(incl, o, 64);
            if (lane >= o) incl += t;
        }
        if (lane == 63) wave_tot[w] = incl;
        __syncthreads();
        int32_t before = 0, total = 0;
        for (int i = 0; i < kSlotThreads / 64; ++i) {
            before += i < w ? wave_tot[i] : 0;
            total += wave_tot[i];
        }
        __syncthreads();
        const int64_t base = carry + before + incl - cnt;
        if (g < G) {
            slot_offsets[g] = (int32_t)min(base, max_slots);
            for (int32_t c = 0; c < cnt; ++c) {
                if (base + c >= max_slots) {
                    bad = 1;
                    break;
                }
                const int32_t t0 = a + c * split;
                ranges[base + c] = int2{t0, min(b, t0 + split)};
            }
        }
        carry += total;
    }
    bad = __syncthreads_or(bad);
    if (tid == 0) {
        slot_offsets[G] = (int32_t)min(carry, max_slots);
        status[kWordSlots] = bad ? 0 : (int32_t)carry;
        status[kWordStatus] = bad ? kStatusPlan : 0;
    }
}

// ---------------------------------------------------------------------------
// The streaming form of the split-K partials, for thin N (at most 32 columns,
// a multiple of 8) and M a multiple of 8.  Items are (split, 256-column M
// tile), M tile fastest, dealt round-robin to the persistent workgroups (one
// per CU), so the workgroups running at one time read neighbouring pieces of
// the same token rows.  A stage is 64 tokens of X and dY.  Eight wavefronts,
// two per SIMD, each own 32 columns of the tile: each thread loads its 16-byte
// pieces into registers two stages ahead (buffer loads whose range check
// supplies the zeros past the stage's last token), writes them to one of two
// LDS buffers, and the MFMA operands come back with the transposing LDS read;
// one workgroup barrier per stage.  The accumulation is the same MFMA sequence
// as splitk_gemm_kernel (16-token steps from the split's first token, rows
// past it zero), so the partials have the same bits; the tile leaves through
// LDS as contiguous 16-byte stores (a split's 256 x N tile is one contiguous
// block of P_s).
constexpr int SM_TM = 256;       // M columns per item
constexpr int SM_TN = 32;        // N columns (one MFMA block, zero-padded past N)
constexpr int SM_TK = 64;        // tokens per stage
constexpr int SM_THREADS = 512;  // 8 wavefronts of 32 M columns
constexpr int SM_XLOADS = SM_TM * SM_TK * 2 / 16 / SM_THREADS;  // 4 pieces of X per thread and stage
constexpr int SM_YPIECES = SM_TN * SM_TK * 2 / 16;               // 256 pieces of dY: threads 0..255
constexpr uint32_t kBufferFlags = 0x00020000u;  // raw buffer (gfx9 resource word 3)
constexpr int kNonTemporal = 2;                 // buffer load cache policy: streaming
constexpr uint32_t kOutOfRange = 0x80000000u;   // a byte offset past every stage's range

struct SmCursor {
    uint32_t item;
    int32_t stage;
    int32_t valid;
};

struct SmStage {
    int64_t t;      // first token
    int32_t rows;   // tokens of the stage
    int32_t last;   // last stage of the split
    int64_t m0;
    int32_t s;      // split
};

__device__ __forceinline__ SmStage sm_stage(const SmCursor& u, int64_t K, int64_t kc, uint32_t mtiles) {
    SmStage g;
    g.s = (int32_t)(u.item / mtiles);
    g.m0 = (int64_t)(u.item % mtiles) * SM_TM;
    const int64_t t_begin = (int64_t)g.s * kc, t_end = min(K, t_begin + kc);
    g.t = t_begin + (int64_t)u.stage * SM_TK;
    g.rows = (int32_t)min((int64_t)SM_TK, t_end - g.t);
    g.last = g.t + SM_TK >= t_end;
    return g;
}

// The stage after u: the next stage of the split, else the worker's next item.
__device__ __forceinline__ SmCursor sm_next(const SmCursor& u, int32_t last, uint32_t P, uint32_t items) {
    SmCursor b = last ? SmCursor{u.item + P, 0, 1} : SmCursor{u.item, u.stage + 1, 1};
    b.valid = u.valid && b.item < items;
    return b;
}

typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

// One stage's pieces of this thread, in registers between their load and their LDS write.
struct SmRegs {
    u32x4v x[SM_XLOADS];
    u32x4v y;
};

__global__ __launch_bounds__(SM_THREADS, 1) void splitk_stream_kernel(const uint16_t* __restrict__ X,
                                                                      const uint16_t* __restrict__ dY, int64_t K,
                                                                      int64_t M, int64_t N, int64_t kc,
                                                                      uint32_t items, uint32_t mtiles,
                                                                      float* __restrict__ out) {
    __shared__ __attribute__((aligned(1024))) uint16_t xs[2][SM_TM * SM_TK];
    __shared__ __attribute__((aligned(1024))) uint16_t ys[2][SM_TN * SM_TK];
    __shared__ __attribute__((aligned(16))) float ot[SM_TM * SM_TN];  // the finished tile, rows of 32
    const uint32_t P = gridDim.x;
    if (blockIdx.x >= items) return;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int i = lane & 31, h = lane >> 5;
    const bool writes_y = tid < SM_YPIECES;  // wavefronts 0..3 write the dY pieces to LDS

    // Piece k of X: position 64 (4 w + k) + lane of the stage, token row p / 32,
    // 16-byte chunk p % 32; its byte offset from the stage's first token row
    // at column m0, and its swizzled LDS element offset.
    int x_row_off[SM_XLOADS], x_col[SM_XLOADS], x_lds[SM_XLOADS];
#pragma unroll
    for (int k = 0; k < SM_XLOADS; ++k) {
        const int pos = 64 * (SM_XLOADS * wv + k) + lane, r = pos / 32, cc = pos % 32;
        x_row_off[k] = (int)(r * M * 2 + 16 * cc);
        x_col[k] = 8 * cc;
        x_lds[k] = lds_at<SM_TM>(r, 8 * cc);
    }
    // Piece tid % 256 of dY: token row (tid % 256) / 4, chunk tid % 4; columns
    // at or past N read zeros.
    const int y_r = (tid & 255) / 4, y_c = 8 * (tid & 3);
    const uint32_t y_off = y_c < N ? (uint32_t)(y_r * N * 2 + 2 * y_c) : kOutOfRange;
    const int y_lds = lds_at<SM_TN>(y_r, y_c);

    const int xoff = operand_offset<SM_TM>(32 * wv);
    const int yoff = operand_offset<SM_TN>(0);

    SmCursor cu{blockIdx.x, 0, 1};  // the stage computed
    SmCursor iu = cu;               // the next stage to load
    // Every call issues the same loads, so the compiler's waits on the
    // registers of a stage count the same instructions on every path; past the
    // worker's last stage every piece is out of range and reads zeros.
    auto issue = [&](SmRegs& rg) {
        const SmStage g = sm_stage(iu, K, kc, mtiles);
        const int32_t rows = iu.valid ? max(g.rows, 0) : 0;
        const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(X + (iu.valid ? g.t * M + g.m0 : 0)), 0, (int)(rows * M * 2), kBufferFlags);
#pragma unroll
        for (int k = 0; k < SM_XLOADS; ++k) {
            const uint32_t off = g.m0 + x_col[k] < M ? (uint32_t)x_row_off[k] : kOutOfRange;
            rg.x[k] = __builtin_bit_cast(u32x4v, __builtin_amdgcn_raw_buffer_load_b128(xr, (int)off, 0, kNonTemporal));
        }
        // every thread loads a dY piece (threads 256.. repeat those of 0..255,
        // from L2) so that every wavefront issues the same loads
        const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(dY + (iu.valid ? g.t * N : 0)), 0, (int)(rows * N * 2), kBufferFlags);
        rg.y = __builtin_bit_cast(u32x4v, __builtin_amdgcn_raw_buffer_load_b128(yr, (int)y_off, 0, 0));
        iu = sm_next(iu, g.last, P, items);
    };
    SmRegs r0, r1;
    issue(r0);
    issue(r1);
    f32x16 acc;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.f;
    int b = 0;  // LDS buffer of the stage computed

    // A finished tile leaves one stage late, after that stage's loads are
    // issued: the vector memory counter retires in issue order, so a load
    // issued after the stores is not known complete before the stores are, and
    // the stage after the stores is waited for only two stages on.
    float* pend_dst = out;
    int pend_pieces = 0;  // 16-byte pieces of the tile waiting in ot (wave-uniform)
    const int q4 = (int)(N / 4);
    float* mine = ot + 32 * wv * SM_TN;  // this wavefront's 32 rows of the tile
    auto flush = [&]() {
        for (int p = lane; p < pend_pieces; p += 64) {
            const int r = p / q4, c = (p % q4) * 4;
            store16_stream(pend_dst + (int64_t)r * N + c, *reinterpret_cast<const u32x4*>(mine + r * SM_TN + c));
        }
        pend_pieces = 0;
    };

    // One stage: its registers go to LDS buffer b, the same registers take the
    // loads of the stage two ahead, and the stage is computed once every
    // wavefront's writes are in.
    auto step = [&](SmRegs& rg) {
        // Buffer b was last read two stages ago; every wavefront has passed the
        // barrier of the stage since, so it is free.
#pragma unroll
        for (int k = 0; k < SM_XLOADS; ++k) *reinterpret_cast<u32x4v*>(xs[b] + x_lds[k]) = rg.x[k];
        if (writes_y) *reinterpret_cast<u32x4v*>(ys[b] + y_lds) = rg.y;
        issue(rg);
        flush();
        lds_barrier();
        const SmStage g = sm_stage(cu, K, kc, mtiles);
        const int ksteps = (g.rows + 15) >> 4;
        for (int ks = 0; ks < ksteps; ++ks) {
            const bf16x8 a = tr_read8(xs[b], xoff + 16 * ks * SM_TM, 4 * SM_TM);
            const bf16x8 bb = tr_read8(ys[b], yoff + 16 * ks * SM_TN, 4 * SM_TN);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bb, acc, 0, 0, 0);
        }
        if (g.last) {
            // Each wavefront writes its rows of the tile to its own part of ot
            // and stores them from there: lane (i, h) holds column i and rows
            // 8 (v / 4) + 4 h + v % 4, and the rows leave as 16-byte pieces (a
            // wavefront's rows are contiguous in P_s).  Only this wavefront
            // touches these rows, and a wavefront's LDS accesses are done in
            // order (the previous tile's stores read ot before these writes),
            // so no workgroup barrier is needed.
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                mine[(8 * (v / 4) + 4 * h + (v % 4)) * SM_TN + i] = acc[v];
                acc[v] = 0.f;
            }
            __builtin_amdgcn_wave_barrier();
            const int64_t m_first = g.m0 + 32 * wv;
            const int rows_out = (int)max((int64_t)0, min(M - m_first, (int64_t)32));
            pend_dst = out + (int64_t)g.s * M * N + m_first * N;
            pend_pieces = rows_out * q4;
        }
        cu = sm_next(cu, g.last, P, items);
        b ^= 1;
    };
    // The worker's stage count, so that the loop below has no exit between
    // its two steps (the compiler's waits then see one order of loads).
    uint32_t stages = 0;
    for (uint32_t it = blockIdx.x; it < items; it += P) {
        const int64_t t_begin = (int64_t)(it / mtiles) * kc, n = min(K, t_begin + kc) - t_begin;
        stages += n > 0 ? (uint32_t)((n + SM_TK - 1) / SM_TK) : 1u;
    }
    for (uint32_t j = 0; j + 2 <= stages; j += 2) {
        step(r0);
        step(r1);
    }
    if (stages & 1) step(r0);
    flush();
}

}  // namespace

hipError_t launch_splitk_gemm(const uint16_t* X, const uint16_t* dY, int64_t K, int64_t M, int64_t N,
                              int32_t splits, float* out, bool atomic, hipStream_t s) {
    const int64_t kc = (K + splits - 1) / splits;
    const int64_t mtiles = (M + BM - 1) / BM, ntiles = (N + BN - 1) / BN;
    const int64_t items = mtiles * ntiles * splits;
    const Launch lc = launch_config();
    // The stream kernel's buffer ranges are 32-bit byte counts of up to 64 token rows.
    if (!atomic && lc.splitk_stream && N <= SM_TN && N % 8 == 0 && M % 8 == 0 && M <= ((int64_t)1 << 23) &&
        (reinterpret_cast<uintptr_t>(X) & 15) == 0 && (reinterpret_cast<uintptr_t>(dY) & 15) == 0 &&
        (reinterpret_cast<uintptr_t>(out) & 15) == 0) {
        const int64_t sm_mtiles = (M + SM_TM - 1) / SM_TM;
        const int64_t sm_items = sm_mtiles * splits;
        int64_t grid = lc.grid_blocks > 0 ? lc.grid_blocks : (int64_t)device_cu_count();
        if (grid > sm_items) grid = sm_items;
        hipLaunchKernelGGL(splitk_stream_kernel, dim3((unsigned)grid), dim3(SM_THREADS), 0, s, X, dY, K, M, N, kc,
                           (uint32_t)sm_items, (uint32_t)sm_mtiles, out);
        return hipGetLastError();
    }
    // three workgroups fit in a CU's LDS; each takes a contiguous range of items
    int64_t grid = lc.grid_blocks > 0 ? lc.grid_blocks : (int64_t)device_cu_count() * 3;
    if (grid > items) grid = items;
    if (atomic)
        hipLaunchKernelGGL(splitk_gemm_kernel<true>, dim3((unsigned)grid), dim3(kGemmThreads), 0, s, X, dY, K, M, N, kc,
                           (uint32_t)items, (uint32_t)mtiles, (uint32_t)ntiles, out, nullptr, nullptr);
    else
        hipLaunchKernelGGL(splitk_gemm_kernel<false>, dim3((unsigned)grid), dim3(kGemmThreads), 0, s, X, dY, K, M, N,
                           kc, (uint32_t)items, (uint32_t)mtiles, (uint32_t)ntiles, out, nullptr, nullptr);
    return hipGetLastError();
}

hipError_t launch_grouped_splitk_gemm(const uint16_t* X, const uint16_t* dY, int64_t K, int64_t M, int64_t N,
                                      const int32_t* group_offsets, int32_t num_groups, int32_t split_tokens,
                                      int64_t max_slots, int32_t* slot_offsets, int2* ranges, int32_t* status,
                                      float* out, hipStream_t s) {
    hipLaunchKernelGGL(grouped_slots_kernel, dim3(1), dim3(kSlotThreads), 0, s, group_offsets, num_groups, K,
                       split_tokens, max_slots, slot_offsets, ranges, status);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t mtiles = (M + BM - 1) / BM, ntiles = (N + BN - 1) / BN;
    const int64_t items_bound = mtiles * ntiles * max_slots;
    const Launch lc = launch_config();
    int64_t grid = lc.grid_blocks > 0 ? lc.grid_blocks : (int64_t)device_cu_count() * 3;
    if (grid > items_bound) grid = items_bound;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(splitk_gemm_kernel<false>, dim3((unsigned)grid), dim3(kGemmThreads), 0, s, X, dY, K, M, N,
                       (int64_t)0, 0u, (uint32_t)mtiles, (uint32_t)ntiles, out, ranges, status);
    return hipGetLastError();
}

hipError_t launch_grouped_reduce(const float* partials, const int32_t* slot_offsets, int64_t max_slots,
                                 int32_t num_groups, int64_t count, float* out, const int32_t* status,
                                 hipStream_t s) {
    if (count == 0 || num_groups == 0) return hipSuccess;
    const bool vec = (count % 4) == 0;
    const int64_t threads = vec ? count / 4 : count;
    const dim3 grid((unsigned)((threads + kReduceThreads - 1) / kReduceThreads), (unsigned)num_groups);
    if (vec)
        hipLaunchKernelGGL(grouped_reduce_kernel<4>, grid, dim3(kReduceThreads), 0, s, partials, slot_offsets,
                           max_slots, count, out, status);
    else
        hipLaunchKernelGGL(grouped_reduce_kernel<1>, grid, dim3(kReduceThreads), 0, s, partials, slot_offsets,
                           max_slots, count, out, status);
    return hipGetLastError();
}

// Workgroups of a split reduce launch (and fingerprint partials it writes).
int64_t splitk_reduce_blocks(int32_t splits, int64_t count) {
    if (count <= 0) return 0;
    const int64_t vectors = (count % 4) == 0 ? count / 4 : count;
    const int64_t chunks = ((int64_t)splits + 7) / 8;
    int64_t lanes = 1;
    if (chunks >= 2 && chunks <= 64) {
        lanes = 2;
        while (lanes < chunks) lanes <<= 1;
    }
    return (vectors * lanes + kReduceThreads - 1) / kReduceThreads;
}

hipError_t launch_splitk_reduce(const float* partials, int32_t splits, int64_t count, float* out, uint64_t* fp_part,
                                hipStream_t s) {
    if (count == 0) return hipSuccess;
    const bool vec = (count % 4) == 0;
    if (fp_part && !vec) return hipErrorInvalidValue;  // the fused fingerprint hashes 16-byte pieces
    const int64_t chunks = ((int64_t)splits + 7) / 8;
    const dim3 grid((unsigned)splitk_reduce_blocks(splits, count)), block(kReduceThreads);
    if (chunks >= 2 && chunks <= 64) {
        // a lane per chunk of 8 splits
        int lanes = 2;
        while (lanes < chunks) lanes <<= 1;
#define DR_RL(V, LN)                                                                                           \
    hipLaunchKernelGGL((splitk_reduce_lanes_kernel<V, LN>), grid, block, 0, s, partials, splits, count, out, \
                       fp_part)
#define DR_RL_V(V)                    \
    switch (lanes) {                  \
        case 2: DR_RL(V, 2); break;   \
        case 4: DR_RL(V, 4); break;   \
        case 8: DR_RL(V, 8); break;   \
        case 16: DR_RL(V, 16); break; \
        case 32: DR_RL(V, 32); break; \
        default: DR_RL(V, 64); break; \
    }
        if (vec) {
            DR_RL_V(4)
        } else {
            DR_RL_V(1)
        }
#undef DR_RL_V
#undef DR_RL
        return hipGetLastError();
    }
    if (vec)
        hipLaunchKernelGGL(splitk_reduce_kernel<4>, grid, block, 0, s, partials, splits, count, out, fp_part);
    else
        hipLaunchKernelGGL(splitk_reduce_kernel<1>, grid, block, 0, s, partials, splits, count, out, fp_part);
    return hipGetLastError();
}

}  // namespace dr
