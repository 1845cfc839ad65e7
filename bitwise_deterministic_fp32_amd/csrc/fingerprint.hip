// Byte fingerprint of a tensor: h = mix(nbytes) + sum_i mix(w_i ^ s_i) mod
// 2^64, where w_i are the little-endian 64-bit words of the bytes (the last one
// zero-padded), s_i = (i + 1) * 0x9e3779b97f4a7c15 is the (i+1)-th state of a
// SplitMix64 generator started at 0, and mix is SplitMix64's finaliser
// (Steele, Lea and Flood, OOPSLA 2014).  Runs are compared byte for byte
// through such fingerprints rather than through printed values
// (bitwise-determinism interview note, "how to verify").  Integer addition is associative, so the two-stage reduction
// below gives the same value for any grid.
#include "internal.h"

namespace dr {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxBlocks = kMaxFingerprintBlocks;

__device__ __forceinline__ uint64_t term(uint64_t w, int64_t i) { return fp_term(w, i); }

constexpr uint64_t kGamma = 0x9e3779b97f4a7c15ull;

__global__ __launch_bounds__(kThreads) void fp_partial_kernel(const unsigned char* __restrict__ data, int64_t nbytes,
                                                              uint64_t* __restrict__ partials) {
    __shared__ uint64_t smem[kThreads / 64];
    const int64_t full = nbytes >> 3;        // complete 8-byte words
    const int64_t words = (nbytes + 7) >> 3;
    const int64_t pairs = full >> 1;          // 16-byte loads
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    uint64_t acc = 0;
    const u32x4* d16 = reinterpret_cast<const u32x4*>(data);
    const bool aligned16 = (reinterpret_cast<uintptr_t>(data) & 15) == 0;
    if (aligned16) {
        int64_t p = (int64_t)blockIdx.x * kThreads + threadIdx.x;
        // The generator states (i + 1) * gamma of the words are carried by
        // wrapping additions (word i of pair p is 2p or 2p + 1), which leaves
        // the two multiplications of the finaliser as the only ones per word.
        const uint64_t step = (uint64_t)(2 * stride) * kGamma;  // state advance of one stride
        uint64_t state = (uint64_t)(2 * p + 1) * kGamma;       // state of word 2p
        // four independent 16-byte loads in flight per lane
        for (; p + 3 * stride < pairs; p += 4 * stride) {
            u32x4 v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(d16 + p + u * stride);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                acc += mix64((((uint64_t)v[u].y << 32) | v[u].x) ^ state);
                acc += mix64((((uint64_t)v[u].w << 32) | v[u].z) ^ (state + kGamma));
                state += step;
            }
        }
        for (; p < pairs; p += stride) {
            const u32x4 v = __builtin_nontemporal_load(d16 + p);
            acc += mix64((((uint64_t)v.y << 32) | v.x) ^ state);
            acc += mix64((((uint64_t)v.w << 32) | v.z) ^ (state + kGamma));
            state += step;
        }
    }
    const int64_t first_single = aligned16 ? 2 * pairs : 0;
    const uint64_t* d8 = reinterpret_cast<const uint64_t*>(data);
    for (int64_t i = first_single + (int64_t)blockIdx.x * kThreads + threadIdx.x; i < words; i += stride) {
        uint64_t w = 0;
        if (i < full) {
            w = d8[i];
        } else {
            for (int64_t b = 0; b < nbytes - 8 * i; ++b) w |= (uint64_t)data[8 * i + b] << (8 * b);
        }
        acc += term(w, i);
    }
    const uint64_t s = block_sum_u64(acc, smem);
    if (threadIdx.x == 0) partials[blockIdx.x] = s;
}

__global__ __launch_bounds__(kThreads) void fp_final_kernel(const uint64_t* __restrict__ partials, int64_t nblocks,
                                                            int64_t nbytes, uint64_t* __restrict__ out) {
    __shared__ uint64_t smem[kThreads / 64];
    uint64_t acc = 0;
    for (int64_t i = threadIdx.x; i < nblocks; i += kThreads) acc += partials[i];
    const uint64_t s = block_sum_u64(acc, smem);
    if (threadIdx.x == 0) *out = s + mix64((uint64_t)nbytes);
}

// One wide workgroup folds up to kWideMax partials (eight loads in flight per
// thread) and adds the length term.
constexpr int kWideThreads = 1024;
constexpr int64_t kWideMax = 64 * kWideThreads;
__global__ __launch_bounds__(kWideThreads) void fp_final_wide_kernel(const uint64_t* __restrict__ partials,
                                                                     int64_t nblocks, int64_t nbytes,
                                                                     uint64_t* __restrict__ out) {
    __shared__ uint64_t smem[kWideThreads / 64];
    uint64_t acc = 0;
    for (int64_t b0 = 0; b0 < nblocks; b0 += 8 * kWideThreads) {
        uint64_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int64_t i = b0 + u * kWideThreads + threadIdx.x;
            v[u] = i < nblocks ? partials[i] : 0;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) acc += v[u];
    }
    const uint64_t s = block_sum_u64(acc, smem);
    if (threadIdx.x == 0) *out = s + mix64((uint64_t)nbytes);
}

}  // namespace

int64_t fingerprint_blocks(int64_t nbytes) {
    const Launch lc = launch_config();
    int64_t b = lc.grid_blocks > 0 ? lc.grid_blocks : (nbytes / 16 + kThreads * 4 - 1) / (kThreads * 4);
    if (b < 1) b = 1;
    if (b > kMaxBlocks) b = kMaxBlocks;
    return b;
}

// Sums groups of kGroup partials per workgroup (four loads in flight per
// thread) into sums[blockIdx.x].
constexpr int kGroup = 4 * kThreads;
__global__ __launch_bounds__(kThreads) void fp_group_kernel(const uint64_t* __restrict__ partials, int64_t nblocks,
                                                            uint64_t* __restrict__ sums) {
    __shared__ uint64_t smem[kThreads / 64];
    const int64_t base = (int64_t)blockIdx.x * kGroup + threadIdx.x;
    uint64_t v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int64_t i = base + u * kThreads;
        v[u] = i < nblocks ? partials[i] : 0;
    }
    const uint64_t s = block_sum_u64(v[0] + v[1] + v[2] + v[3], smem);
    if (threadIdx.x == 0) sums[blockIdx.x] = s;
}

int64_t fingerprint_group_count(int64_t nblocks) { return (nblocks + kGroup - 1) / kGroup; }

hipError_t launch_fingerprint_final(const uint64_t* block_partials, int64_t nblocks, int64_t nbytes, uint64_t* out,
                                    uint64_t* group_sums, hipStream_t s) {
    if (nblocks > kGroup && nblocks <= kWideMax) {
        hipLaunchKernelGGL(fp_final_wide_kernel, dim3(1), dim3(kWideThreads), 0, s, block_partials, nblocks, nbytes,
                           out);
        return hipGetLastError();
    }
    if (nblocks > kGroup && group_sums) {
        // two levels: many workgroups fold the partials, one folds their sums
        const int64_t groups = fingerprint_group_count(nblocks);
        hipLaunchKernelGGL(fp_group_kernel, dim3((unsigned)groups), dim3(kThreads), 0, s, block_partials, nblocks,
                           group_sums);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        block_partials = group_sums;
        nblocks = groups;
    }
    hipLaunchKernelGGL(fp_final_kernel, dim3(1), dim3(kThreads), 0, s, block_partials, nblocks, nbytes, out);
    return hipGetLastError();
}

// An incremental update: the reduce kernels that rewrite destination pieces
// leave the change of those pieces' terms (new minus old), one sum per
// workgroup; the fingerprint of the whole tensor moves by their total.
__global__ __launch_bounds__(kWideThreads) void fp_update_kernel(const uint64_t* __restrict__ parts, int64_t nparts,
                                                                 const int32_t* __restrict__ status,
                                                                 uint64_t* __restrict__ hash) {
    __shared__ uint64_t smem[kWideThreads / 64];
    if (status[kWordStatus] != 0) return;  // the call failed closed: its destination and hash stay as they were
    uint64_t acc = 0;
    for (int64_t i = threadIdx.x; i < nparts; i += kWideThreads) acc += parts[i];
    const uint64_t s = block_sum_u64(acc, smem);
    if (threadIdx.x == 0) *hash += s;
}

hipError_t launch_fingerprint_update(const uint64_t* parts, int64_t nparts, const int32_t* status, uint64_t* hash,
                                     hipStream_t s) {
    hipLaunchKernelGGL(fp_update_kernel, dim3(1), dim3(kWideThreads), 0, s, parts, nparts, status, hash);
    return hipGetLastError();
}

hipError_t launch_fingerprint(const void* data, int64_t nbytes, uint64_t* out, uint64_t* block_partials,
                              hipStream_t s) {
    const int64_t nb = fingerprint_blocks(nbytes);
    hipLaunchKernelGGL(fp_partial_kernel, dim3((unsigned)nb), dim3(kThreads), 0, s,
                       reinterpret_cast<const unsigned char*>(data), nbytes, block_partials);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_fingerprint_final(block_partials, nb, nbytes, out, nullptr, s);
}

}  // namespace dr
