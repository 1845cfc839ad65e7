// The deliberately nondeterministic index_add baseline: every contribution row
// is added into its destination row with hardware fp32 atomics, so the order
// of the adds into one element is whatever order they arrive in.  This is the
// default path of the pages (Megatron-LM op catalog, determinism reference
// section 3.1: atomic scatter_add_ / embedding backward; DeepSeek-V4 book
// ch. 9, "atomicAdd" glossary entry), kept as the overhead reference.
#include "internal.h"

namespace dr {
namespace {

constexpr int kThreads = 256;

template <dr_dtype DT>
__global__ __launch_bounds__(kThreads) void index_add_atomic_kernel(float* __restrict__ out, int32_t num_dests,
                                                                    int64_t H, const void* __restrict__ src,
                                                                    int64_t n, const int32_t* __restrict__ index,
                                                                    int32_t* dev_status, int64_t pieces) {
    constexpr int E = Vec<DT>::kElems;
    constexpr int kElemBytes = DT == DR_BF16 ? 2 : 4;
    // the host keeps n * pieces below 2^32
    const uint32_t g = blockIdx.x * kThreads + threadIdx.x;
    const uint32_t i = g / (uint32_t)pieces;
    const int64_t piece = g - i * (uint32_t)pieces;
    if (i >= n) return;
    const int32_t d = index[i];
    if (d < 0 || d >= num_dests) {
        if (dev_status && piece == 0) atomicOr(dev_status, kStatusIndex);
        return;
    }
    float v[E];
    Vec<DT>::widen(load16(reinterpret_cast<const char*>(src) + ((int64_t)i * H + piece * E) * kElemBytes), v);
    float* o = out + (int64_t)d * H + piece * E;
#pragma unroll
    for (int e = 0; e < E; ++e) unsafeAtomicAdd(o + e, v[e]);
}

}  // namespace

hipError_t launch_index_add_atomic(float* out, int32_t num_dests, int64_t hidden, const void* src, dr_dtype dt,
                                   int64_t n, const int32_t* index, int32_t* dev_status, hipStream_t s) {
    if (n == 0) return hipSuccess;
    const int64_t pieces = dt == DR_BF16 ? hidden / 8 : hidden / 4;
    const int64_t threads = n * pieces;
    const dim3 grid((unsigned)((threads + kThreads - 1) / kThreads));
    if (dt == DR_BF16)
        hipLaunchKernelGGL(index_add_atomic_kernel<DR_BF16>, grid, dim3(kThreads), 0, s, out, num_dests, hidden, src,
                           n, index, dev_status, pieces);
    else
        hipLaunchKernelGGL(index_add_atomic_kernel<DR_F32>, grid, dim3(kThreads), 0, s, out, num_dests, hidden, src, n,
                           index, dev_status, pieces);
    return hipGetLastError();
}

}  // namespace dr
