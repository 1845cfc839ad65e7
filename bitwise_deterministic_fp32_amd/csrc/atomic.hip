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

// One wavefront per (contribution row, slice of 64*E columns).  Lane l reads
// the 16 bytes of columns [E*l, E*l + E) of the slice with one vector load
// (the access the ordered kernels use), the wavefront re-deals the widened
// values through LDS so that lane l holds columns l + 64*e, and every atomic
// instruction then covers 64 consecutive elements (two or four whole cache
// lines).  So the baseline reads and adds as efficiently as the hardware
// allows; only the order of the adds is left to the arrival order.
template <dr_dtype DT>
__global__ __launch_bounds__(kThreads) void index_add_atomic_kernel(float* __restrict__ out, int32_t num_dests,
                                                                    int64_t H, const void* __restrict__ src,
                                                                    int64_t n, const int32_t* __restrict__ index,
                                                                    int32_t* dev_status, int64_t slices) {
    constexpr int E = Vec<DT>::kElems;
    constexpr int kElemBytes = DT == DR_BF16 ? 2 : 4;
    __shared__ float stage[kThreads / 64][64 * E];
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    // the host keeps n * slices below 2^32
    const uint32_t wave = blockIdx.x * (kThreads / 64) + w;
    const uint32_t i = wave / (uint32_t)slices;
    bool live = i < n;
    const uint32_t slice = live ? wave - i * (uint32_t)slices : 0;
    const int32_t d = live ? index[i] : 0;
    if (live && (d < 0 || d >= num_dests)) {
        if (dev_status && lane == 0 && slice == 0) atomicOr(dev_status, kStatusIndex);
        live = false;
    }
    // hidden is a multiple of E, so a lane's 16 bytes lie wholly inside or wholly past the row
    const int64_t cv = (int64_t)slice * 64 * E + (int64_t)lane * E;
    if (live && cv < H) {
        const char* row = reinterpret_cast<const char*>(src) + (int64_t)i * H * kElemBytes;
        float v[E];
        Vec<DT>::widen(load16_stream(row + cv * kElemBytes), v);
#pragma unroll
        for (int e = 0; e < E; ++e) stage[w][lane * E + e] = v[e];
    }
    __syncthreads();
    if (!live) return;
    float* o = out + (int64_t)d * H;
    const int64_t c0 = (int64_t)slice * 64 * E + lane;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int64_t c = c0 + 64 * e;
        if (c < H) unsafeAtomicAdd(o + c, stage[w][lane + 64 * e]);
    }
}

}  // namespace

hipError_t launch_index_add_atomic(float* out, int32_t num_dests, int64_t hidden, const void* src, dr_dtype dt,
                                   int64_t n, const int32_t* index, int32_t* dev_status, hipStream_t s) {
    if (n == 0) return hipSuccess;
    const int64_t per_wave = 64 * (dt == DR_BF16 ? 8 : 4);
    const int64_t slices = (hidden + per_wave - 1) / per_wave;
    const int64_t waves = n * slices;
    const dim3 grid((unsigned)((waves + kThreads / 64 - 1) / (kThreads / 64)));
    if (dt == DR_BF16)
        hipLaunchKernelGGL(index_add_atomic_kernel<DR_BF16>, grid, dim3(kThreads), 0, s, out, num_dests, hidden, src,
                           n, index, dev_status, slices);
    else
        hipLaunchKernelGGL(index_add_atomic_kernel<DR_F32>, grid, dim3(kThreads), 0, s, out, num_dests, hidden, src, n,
                           index, dev_status, slices);
    return hipGetLastError();
}

}  // namespace dr
