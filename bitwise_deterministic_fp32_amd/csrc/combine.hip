// MoE token combine (unpermute) in the defined order, and its atomicAdd
// baseline.
//
// out[t] = T over the token's k contributions fl32(gate * row), taken in
// ascending row order.  With the expert-major layout that the dispatch sort
// produces, that is expert-id order.  It is the same for every expert-parallel
// size, since the order key is the row (expert), not the rank that computed
// it.  This is the sorted-order merge of the DeepSeek-V4 MoE backward (ch. 9,
// section 3.2) and the unpermute row of the Megatron-LM op catalog
// (determinism reference, section 3.1).
//
// One wavefront owns one token and a slice of 64 x 16 bytes of its columns.
// The k slots are ranked by row id with wave-uniform data.  Then each lane
// issues all k row loads of the first chunk (up to 8 x 16 B in flight) and
// sums the products left to right.  The output is written exactly once; the
// same data never passes through an atomic, and no memset is needed.
#include "internal.h"

namespace dr {
namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / 64;
// k <= 8 uses 8-wavefront workgroups (measured a little faster than 4 or 16
// at the MoE shape, and half as many fingerprint partials to fold as 4).
// Larger k keeps 4: it needs more registers per lane.
constexpr int kThreadsK8 = 512;

__device__ __forceinline__ int32_t uniform_lane(int32_t v, int lane) {
    return __builtin_amdgcn_readlane(v, lane);
}

// The work of one wavefront: token t, column slice `slice`.  Returns this
// lane's sum of fingerprint terms of the bytes it stored (FP), else 0.
template <dr_dtype DT, int KMAX, bool FP>
__device__ __forceinline__ uint64_t combine_token(const void* __restrict__ rows, int64_t num_rows, int64_t H,
                                                  const int32_t* __restrict__ row_of, const float* __restrict__ gates,
                                                  int k, float* __restrict__ out, int32_t* dev_status, int64_t t,
                                                  uint32_t slice) {
    using PC = Piece<DT>;
    constexpr int P = PC::kPieces;
    constexpr int kElemBytes = DT == DR_BF16 ? 2 : 4;
    constexpr int64_t W = 64 * 4 * P;  // columns of one wavefront slice
    const int lane = threadIdx.x & 63;

    // piece p of this lane: columns col[p] .. col[p]+3; pieces of a wavefront
    // are 256 columns apart so each load and store instruction is contiguous
    int64_t col[P], lcol[P];
    bool active[P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
        col[p] = (int64_t)slice * W + p * 256 + 4 * lane;
        active[p] = col[p] < H;
        lcol[p] = active[p] ? col[p] : 0;  // idle lanes read a valid piece
    }
    float* orow = out + t * H;

    int32_t rid = INT32_MAX;
    float g = 0.f;
    if (lane < k) {
        rid = row_of[t * k + lane];
        g = gates[t * k + lane];
    }
    const bool bad = lane < k && (rid < 0 || rid >= num_rows);
    if (__ballot(bad) != 0) {
        // fail closed: never read outside rows; the token's output is poisoned
        const uint32_t nan = 0x7FC00000u;
        uint64_t hash = 0;
#pragma unroll
        for (int p = 0; p < P; ++p)
            if (active[p]) {
                store16(orow + col[p], u32x4{nan, nan, nan, nan});
                if (FP) {
                    const int64_t i0 = (t * H + col[p]) >> 1;  // 8-byte word index
                    const uint64_t w = ((uint64_t)nan << 32) | nan;
                    hash += fp_term(w, i0) + fp_term(w, i0 + 1);
                }
            }
        if (dev_status && lane == 0 && slice == 0) atomicOr(dev_status, kStatusIndex);
        return hash;
    }
    const char* rb = reinterpret_cast<const char*>(rows);
    const int64_t row_bytes = H * kElemBytes;

    // rank of each slot by (row, slot)
    int rank = 0;
    for (int i = 0; i < k; ++i) {
        const int32_t ri = __shfl(rid, i, 64);
        rank += (ri < rid) || (ri == rid && i < lane);
    }
    if (lane >= k) rank = 64 + lane;  // never selected

    float res[P][4];
    if (KMAX <= 8) {
        // one chunk: left to right over the sorted slots.  Slots past k reload
        // the last slot's row (a cache hit) so that all loads issue together;
        // they are not added.
        typename PC::Raw raw[8][P];
        float gq[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const uint64_t sel = __ballot(rank == min(q, k - 1));
            const int src_lane = __builtin_ctzll(sel);
            const int32_t r = uniform_lane(rid, src_lane);
            gq[q] = __int_as_float(uniform_lane(__float_as_int(g), src_lane));
#pragma unroll
            for (int p = 0; p < P; ++p) raw[q][p] = PC::load_stream(rb + (int64_t)r * row_bytes, lcol[p]);
        }
#pragma unroll
        for (int p = 0; p < P; ++p) {
            float y[4];
            PC::widen(raw[0][p], y);
#pragma unroll
            for (int e = 0; e < 4; ++e) res[p][e] = gq[0] * y[e];
#pragma unroll
            for (int q = 1; q < 8; ++q) {
                PC::widen(raw[q][p], y);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float prod = gq[q] * y[e];  // rounded product, then the add
                    const float a = res[p][e] + prod;
                    res[p][e] = q < k ? a : res[p][e];
                }
            }
        }
    } else {
        // up to 8 chunks of 8; chunk sums padded with -0.0 and paired by
        // stride doubling, which is the tree T for any chunk count <= 8
        float cs[8][P][4];
#pragma unroll
        for (int c = 0; c < 8; ++c)
#pragma unroll
            for (int p = 0; p < P; ++p)
#pragma unroll
                for (int e = 0; e < 4; ++e) cs[c][p][e] = neg_zero();
        const int nchunks = (k + 7) >> 3;
        for (int c = 0; c < nchunks; ++c) {
            const int m = min(8, k - 8 * c);
            typename PC::Raw raw[8][P];
            float gq[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint64_t sel = __ballot(rank == 8 * c + min(j, m - 1));
                const int src_lane = __builtin_ctzll(sel);
                const int32_t r = uniform_lane(rid, src_lane);
                gq[j] = __int_as_float(uniform_lane(__float_as_int(g), src_lane));
#pragma unroll
                for (int p = 0; p < P; ++p) raw[j][p] = PC::load_stream(rb + (int64_t)r * row_bytes, lcol[p]);
            }
            float s[P][4];
#pragma unroll
            for (int p = 0; p < P; ++p) {
                float y[4];
                PC::widen(raw[0][p], y);
#pragma unroll
                for (int e = 0; e < 4; ++e) s[p][e] = gq[0] * y[e];
#pragma unroll
                for (int j = 1; j < 8; ++j) {
                    PC::widen(raw[j][p], y);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float prod = gq[j] * y[e];
                        const float a = s[p][e] + prod;
                        s[p][e] = j < m ? a : s[p][e];
                    }
                }
            }
#pragma unroll
            for (int cc = 0; cc < 8; ++cc) {
                if (cc == c) {
#pragma unroll
                    for (int p = 0; p < P; ++p)
#pragma unroll
                        for (int e = 0; e < 4; ++e) cs[cc][p][e] = s[p][e];
                }
            }
        }
#pragma unroll
        for (int p = 0; p < P; ++p) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float a = cs[0][p][e] + cs[1][p][e], b = cs[2][p][e] + cs[3][p][e];
                const float c2 = cs[4][p][e] + cs[5][p][e], d = cs[6][p][e] + cs[7][p][e];
                const float ab = a + b, cd = c2 + d;
                res[p][e] = ab + cd;
            }
        }
    }
    uint64_t hash = 0;
#pragma unroll
    for (int p = 0; p < P; ++p)
        if (active[p]) {
            const u32x4 v{__float_as_uint(res[p][0]), __float_as_uint(res[p][1]), __float_as_uint(res[p][2]),
                          __float_as_uint(res[p][3])};
            store16_stream(orow + col[p], v);
            if (FP) {
                // the fingerprint's terms of the two 8-byte words just stored
                const int64_t i0 = (t * H + col[p]) >> 1;
                hash += fp_term(((uint64_t)v.y << 32) | v.x, i0) + fp_term(((uint64_t)v.w << 32) | v.z, i0 + 1);
            }
        }
    return hash;
}

// One wavefront per (token, column slice).  With FP, the workgroup also sums
// the fingerprint terms of what it stored into fp_partials[blockIdx.x]
// (wrapping addition, so the total does not depend on the grid).
template <dr_dtype DT, int KMAX, bool FP, int THREADS>
__global__ __launch_bounds__(THREADS) void combine_kernel(const void* __restrict__ rows, int64_t num_rows, int64_t H,
                                                           const int32_t* __restrict__ row_of,
                                                           const float* __restrict__ gates, int64_t T, int k,
                                                           float* __restrict__ out, int32_t* dev_status,
                                                           int64_t slices, uint64_t* __restrict__ fp_partials) {
    // the host keeps T * slices below 2^32
    const uint32_t wave = blockIdx.x * (THREADS / 64) + (threadIdx.x >> 6);
    const uint32_t t32 = wave / (uint32_t)slices;
    uint64_t hash = 0;
    if (t32 < T) {  // whole wavefront
        const int64_t t = t32;
        hash = combine_token<DT, KMAX, FP>(rows, num_rows, H, row_of, gates, k, out, dev_status, t,
                                           wave - t32 * (uint32_t)slices);
    }
    if (FP) {
        __shared__ uint64_t smem[THREADS / 64];
        const uint64_t s = block_sum_u64(hash, smem);
        if (threadIdx.x == 0) fp_partials[blockIdx.x] = s;
    }
}

// The baseline: one wavefront per (token, slot, slice of 64*E columns), so
// the k contributions of an output element come from k different wavefronts
// and are added by hardware fp32 atomics in whatever order they arrive (the
// scatter_add_ pattern over permuted rows).  Each lane reads 16 bytes with one
// vector load; after an exchange through LDS, lane l holds columns l + 64*e,
// so every atomic instruction covers 64 consecutive elements.
template <dr_dtype DT>
__global__ __launch_bounds__(kThreads) void combine_atomic_kernel(const void* __restrict__ rows, int64_t num_rows,
                                                                  int64_t H, const int32_t* __restrict__ row_of,
                                                                  const float* __restrict__ gates, int64_t T, int k,
                                                                  float* __restrict__ out, int32_t* dev_status,
                                                                  int64_t slices) {
    constexpr int E = Vec<DT>::kElems;
    constexpr int kElemBytes = DT == DR_BF16 ? 2 : 4;
    __shared__ float stage[kWavesPerBlock][64 * E];
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    // the host keeps T * k * slices below 2^32
    const uint32_t wave = blockIdx.x * kWavesPerBlock + w;
    const uint32_t a = wave / (uint32_t)slices;  // assignment index t*k + j
    bool live = a < (uint64_t)T * k;
    const uint32_t slice = live ? wave - a * (uint32_t)slices : 0;
    const int32_t r = live ? row_of[a] : 0;
    if (live && (r < 0 || r >= num_rows)) {
        if (dev_status && lane == 0 && slice == 0) atomicOr(dev_status, kStatusIndex);
        live = false;
    }
    // one 16-byte load per lane, re-dealt through LDS so that each atomic
    // instruction covers 64 consecutive output elements
    const int64_t cv = (int64_t)slice * 64 * E + (int64_t)lane * E;
    if (live && cv < H) {
        const char* row = reinterpret_cast<const char*>(rows) + (int64_t)r * H * kElemBytes;
        float y[E];
        Vec<DT>::widen(load16_stream(row + cv * kElemBytes), y);
#pragma unroll
        for (int e = 0; e < E; ++e) stage[w][lane * E + e] = y[e];
    }
    __syncthreads();
    if (!live) return;
    const int64_t t = a / (uint32_t)k;
    const float g = gates[a];
    float* o = out + t * H;
    const int64_t c0 = (int64_t)slice * 64 * E + lane;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int64_t c = c0 + 64 * e;
        if (c < H) {
            const float p = g * stage[w][lane + 64 * e];
            unsafeAtomicAdd(o + c, p);
        }
    }
}

template <dr_dtype DT>
hipError_t launch_dt(const void* rows, int64_t num_rows, int64_t H, const int32_t* row_of, const float* gates,
                     int64_t T, int32_t k, float* out, int32_t* dev_status, bool atomic, uint64_t* fp_partials,
                     hipStream_t s) {
    constexpr int E = Vec<DT>::kElems;
    const int64_t pieces = H / E;
    const int64_t slices = (pieces + 63) / 64;
    if (atomic) {
        const int64_t waves = T * k * slices;
        const dim3 grid((unsigned)((waves + kWavesPerBlock - 1) / kWavesPerBlock));
        hipLaunchKernelGGL(combine_atomic_kernel<DT>, grid, dim3(kThreads), 0, s, rows, num_rows, H, row_of, gates, T,
                           k, out, dev_status, slices);
        return hipGetLastError();
    }
    const int64_t waves = T * slices;
#define DR_COMBINE(KM, FPV, TH)                                                                                 \
    hipLaunchKernelGGL((combine_kernel<DT, KM, FPV, TH>), dim3((unsigned)((waves + TH / 64 - 1) / (TH / 64))), \
                       dim3(TH), 0, s, rows, num_rows, H, row_of, gates, T, k, out, dev_status, slices, fp_partials)
    if (fp_partials) {
        if (k <= 8) DR_COMBINE(8, true, kThreadsK8);
        else DR_COMBINE(64, true, kThreads);
    } else {
        if (k <= 8) DR_COMBINE(8, false, kThreadsK8);
        else DR_COMBINE(64, false, kThreads);
    }
#undef DR_COMBINE
    return hipGetLastError();
}

}  // namespace

int64_t combine_fp_blocks(dr_dtype dt, int64_t hidden, int64_t T, int32_t k) {
    const int64_t per_wave = 64 * (dt == DR_BF16 ? 8 : 4);
    const int64_t slices = (hidden + per_wave - 1) / per_wave;
    const int64_t waves_per_block = (k <= 8 ? kThreadsK8 : kThreads) / 64;
    return (T * slices + waves_per_block - 1) / waves_per_block;
}

hipError_t launch_combine(const void* rows, dr_dtype dt, int64_t num_rows, int64_t hidden, const int32_t* row_of,
                          const float* gates, int64_t T, int32_t k, float* out, int32_t* dev_status, bool atomic,
                          uint64_t* fp_partials, hipStream_t s) {
    if (T == 0) return hipSuccess;
    if (dt == DR_BF16)
        return launch_dt<DR_BF16>(rows, num_rows, hidden, row_of, gates, T, k, out, dev_status, atomic, fp_partials, s);
    return launch_dt<DR_F32>(rows, num_rows, hidden, row_of, gates, T, k, out, dev_status, atomic, fp_partials, s);
}

}  // namespace dr
