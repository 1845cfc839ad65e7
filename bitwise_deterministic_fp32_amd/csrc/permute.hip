// Dispatch-side stable permute of the MoE layer: token rows copied into the
// expert-major order the dispatch sort defines.
//
// out[r] = rows[perm[r] / k], where perm is dr_sort_by_dest's permutation of
// the T*k (token, slot) assignments by expert (ties by token, then slot).
// This is the gather that puts each expert's tokens contiguously, in token
// order, before the expert GEMMs (DeepSeek-V4 book, ch. 9, section 3.2: tokens
// sorted by (expert_id, original_token_id)).  It moves bytes only, so it is
// exact; the order it produces is what makes the later combine and the
// grouped weight gradient independent of the expert-parallel layout.
//
// One wavefront copies one output row in 16-byte pieces (four in flight per
// lane); the output is written once, with streaming stores.  A token row is
// read k times.  Given the sort's inverse permutation, wavefront w takes
// output row inv[w] (w = t*k + j in token order), so the k copies of a token
// are made by neighbouring wavefronts and its row is read from cache rather
// than from HBM k times; the wavefront checks perm[inv[w]] == w, so every
// output row is still the one perm assigns and is written once.
#include "internal.h"

namespace dr {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

__global__ __launch_bounds__(kThreads) void permute_rows_kernel(const unsigned char* __restrict__ rows,
                                                                int64_t row_bytes, int64_t num_rows,
                                                                const int32_t* __restrict__ perm,
                                                                const int32_t* __restrict__ inv, int64_t n,
                                                                uint32_t k, unsigned char* __restrict__ out,
                                                                int32_t* dev_status) {
    const int64_t w = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (w >= n) return;  // whole wavefront
    const int lane = threadIdx.x & 63;
    int64_t r = w;
    bool ok = true;
    if (inv) {
        r = inv[w];
        ok = r >= 0 && r < n && perm[r] == (int32_t)w;
    }
    const int32_t p = ok ? perm[r] : -1;
    const int64_t src = p >= 0 ? (int64_t)((uint32_t)p / k) : -1;  // 32-bit division
    if (src < 0 || src >= num_rows) {
        // fail closed: the row is not written
        if (dev_status && lane == 0) atomicOr(dev_status, kStatusIndex);
        return;
    }
    const unsigned char* s = rows + src * row_bytes;
    unsigned char* d = out + r * row_bytes;
    const int64_t pieces = row_bytes >> 4;
    for (int64_t c0 = lane; c0 < pieces; c0 += 4 * 64) {
        u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t c = c0 + 64 * u;
            v[u] = c < pieces ? load16(s + (c << 4)) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t c = c0 + 64 * u;
            if (c < pieces) store16_stream(d + (c << 4), v[u]);
        }
    }
}

}  // namespace

hipError_t launch_permute_rows(const void* rows, int64_t row_bytes, int64_t num_rows, const int32_t* perm,
                               const int32_t* inv_perm, int64_t n, int32_t k, void* out, int32_t* dev_status,
                               hipStream_t s) {
    if (n == 0) return hipSuccess;
    const dim3 grid((unsigned)((n + kWaves - 1) / kWaves));
    hipLaunchKernelGGL(permute_rows_kernel, grid, dim3(kThreads), 0, s, static_cast<const unsigned char*>(rows),
                       row_bytes, num_rows, perm, inv_perm, n, (uint32_t)k, static_cast<unsigned char*>(out),
                       dev_status);
    return hipGetLastError();
}

}  // namespace dr
