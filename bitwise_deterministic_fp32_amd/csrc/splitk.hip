// Split-K thin contraction dW = X^T dY into private per-split buffers, and the
// ordered reduce over split ids.
//
// The DeepSeek-V4 mHC backward (ch. 9, section 3.3) has an output dimension of
// only 24.  It must split the contraction, and it keeps one buffer per split,
// reduced afterwards by a dedicated kernel in split-id order.  Here:
//   splitk_gemm: one workgroup per (split, 64-row M tile, 32-column N tile).
//     Tokens of the split are staged through LDS in rows of 64, and each of the
//     two wavefronts accumulates a 32x32 tile with the bf16 MFMA
//     v_mfma_f32_32x32x16_bf16, in token order, into fp32.  A partial depends
//     only on (split, m, n): not on the grid, the M/N tiling or other columns.
//     The HBM stream is X (read once); the MFMA work is small beside it.
//   splitk_reduce: out[e] = T(P_0[e], ..., P_{S-1}[e]); chunks of 8 splits left
//     to right, then the pairwise tree, one thread per 4 consecutive elements.
// The atomic baseline runs the same tile code and adds each split's tile into
// out with hardware fp32 atomics.
#include "internal.h"

namespace dr {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 64;  // M rows per workgroup (two 32-row wavefront tiles)
constexpr int BN = 32;  // N columns per workgroup
constexpr int KT = 64;  // tokens per LDS stage
constexpr int kGemmThreads = 128;
// Row strides (in bf16) padded so that the two half-wavefronts of a transposed
// operand read (rows 8 apart) fall in different LDS banks.
constexpr int XS = BM + 4;
constexpr int YS = BN + 4;

__device__ __forceinline__ __bf16 as_bf16(uint16_t b) { return __builtin_bit_cast(__bf16, b); }

template <bool ATOMIC>
__global__ __launch_bounds__(kGemmThreads) void splitk_gemm_kernel(const uint16_t* __restrict__ X,
                                                                   const uint16_t* __restrict__ dY, int64_t K,
                                                                   int64_t M, int64_t N, int64_t kc,
                                                                   float* __restrict__ out) {
    __shared__ uint16_t xs[KT * XS];
    __shared__ uint16_t ys[KT * YS];
    const int s = blockIdx.z;
    const int64_t m0 = (int64_t)blockIdx.x * BM;
    const int64_t n0 = (int64_t)blockIdx.y * BN;
    const int64_t t_begin = (int64_t)s * kc;
    const int64_t t_end = min(K, t_begin + kc);
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const bool m_vec_ok = (M % 8) == 0;

    f32x16 acc;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.f;

    for (int64_t t0 = t_begin; t0 < t_end; t0 += KT) {
        // X[t0 .. t0+KT) x [m0 .. m0+BM) -> xs, zero outside the split / matrix
        for (int p = tid; p < KT * (BM / 8); p += kGemmThreads) {
            const int r = p / (BM / 8), c8 = (p % (BM / 8)) * 8;
            const int64_t t = t0 + r, m = m0 + c8;
            uint16_t v8[8];
            if (t < t_end && m_vec_ok && m + 8 <= M) {
                const u32x4 raw = load16(X + t * M + m);
                v8[0] = raw.x & 0xFFFF; v8[1] = raw.x >> 16;
                v8[2] = raw.y & 0xFFFF; v8[3] = raw.y >> 16;
                v8[4] = raw.z & 0xFFFF; v8[5] = raw.z >> 16;
                v8[6] = raw.w & 0xFFFF; v8[7] = raw.w >> 16;
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) v8[e] = (t < t_end && m + e < M) ? X[t * M + m + e] : (uint16_t)0;
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) xs[r * XS + c8 + e] = v8[e];
        }
        for (int p = tid; p < KT * BN; p += kGemmThreads) {
            const int r = p / BN, c = p % BN;
            const int64_t t = t0 + r, n = n0 + c;
            ys[r * YS + c] = (t < t_end && n < N) ? dY[t * N + n] : (uint16_t)0;
        }
        __syncthreads();
        const int i = lane & 31, g = lane >> 5;
#pragma unroll
        for (int kk = 0; kk < KT; kk += 16) {
            bf16x8 a, b;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                a[e] = as_bf16(xs[(kk + 8 * g + e) * XS + wv * 32 + i]);
                b[e] = as_bf16(ys[(kk + 8 * g + e) * YS + i]);
            }
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
        }
        __syncthreads();
    }

    // accumulator layout of a 32x32 MFMA tile: lane holds column (lane % 32)
    // and rows 8*(v/4) + 4*(lane/32) + (v%4) for v = 0..15
    const int j = lane & 31, g = lane >> 5;
    const int64_t n = n0 + j;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int64_t m = m0 + wv * 32 + 8 * (v / 4) + 4 * g + (v % 4);
        if (m < M && n < N) {
            if (ATOMIC) unsafeAtomicAdd(out + m * N + n, acc[v]);
            else out[(int64_t)s * M * N + m * N + n] = acc[v];
        }
    }
}

constexpr int kReduceThreads = 256;
constexpr int kReduceDepth = 24;  // chunk sums per element < 2^24 (splits < 2^27)

template <int VEC>
__global__ __launch_bounds__(kReduceThreads) void splitk_reduce_kernel(const float* __restrict__ P, int S,
                                                                       int64_t count, float* __restrict__ out) {
    const int64_t e0 = ((int64_t)blockIdx.x * kReduceThreads + threadIdx.x) * VEC;
    if (e0 >= count) return;
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

}  // namespace

hipError_t launch_splitk_gemm(const uint16_t* X, const uint16_t* dY, int64_t K, int64_t M, int64_t N,
                              int32_t splits, float* out, bool atomic, hipStream_t s) {
    const int64_t kc = (K + splits - 1) / splits;
    const dim3 grid((unsigned)((M + BM - 1) / BM), (unsigned)((N + BN - 1) / BN), (unsigned)splits);
    if (atomic)
        hipLaunchKernelGGL(splitk_gemm_kernel<true>, grid, dim3(kGemmThreads), 0, s, X, dY, K, M, N, kc, out);
    else
        hipLaunchKernelGGL(splitk_gemm_kernel<false>, grid, dim3(kGemmThreads), 0, s, X, dY, K, M, N, kc, out);
    return hipGetLastError();
}

hipError_t launch_splitk_reduce(const float* partials, int32_t splits, int64_t count, float* out, hipStream_t s) {
    if (count == 0) return hipSuccess;
    const bool vec = (count % 4) == 0;
    const int64_t threads = vec ? count / 4 : count;
    const dim3 grid((unsigned)((threads + kReduceThreads - 1) / kReduceThreads));
    if (vec)
        hipLaunchKernelGGL(splitk_reduce_kernel<4>, grid, dim3(kReduceThreads), 0, s, partials, splits, count, out);
    else
        hipLaunchKernelGGL(splitk_reduce_kernel<1>, grid, dim3(kReduceThreads), 0, s, partials, splits, count, out);
    return hipGetLastError();
}

}  // namespace dr
