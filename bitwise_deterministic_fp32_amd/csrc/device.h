// Device helpers shared by the HIP kernels of libdetreduce (loads, stores,
// widening, the fingerprint's terms, wavefront sums).  Included by internal.h
// when compiling device code.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "detreduce.h"

namespace dr {

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16 bytes of row data widened to fp32: 8 bf16 values or 4 fp32 values.
template <dr_dtype DT>
struct Vec;

template <>
struct Vec<DR_BF16> {
    static constexpr int kElems = 8;
    __device__ __forceinline__ static void widen(const u32x4& raw, float (&v)[8]) {
        v[0] = bf16_lo(raw.x); v[1] = bf16_hi(raw.x);
        v[2] = bf16_lo(raw.y); v[3] = bf16_hi(raw.y);
        v[4] = bf16_lo(raw.z); v[5] = bf16_hi(raw.z);
        v[6] = bf16_lo(raw.w); v[7] = bf16_hi(raw.w);
    }
};

template <>
struct Vec<DR_F32> {
    static constexpr int kElems = 4;
    __device__ __forceinline__ static void widen(const u32x4& raw, float (&v)[4]) {
        v[0] = __uint_as_float(raw.x); v[1] = __uint_as_float(raw.y);
        v[2] = __uint_as_float(raw.z); v[3] = __uint_as_float(raw.w);
    }
};

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// A lane's unit of row data: 4 consecutive columns, widened to fp32.  bf16
// rows are read as 8-byte pieces and fp32 rows as 16-byte pieces.  A lane owns
// kPieces pieces kSpan columns apart, so that both the loads and the 16-byte
// fp32 stores of a lane group cover contiguous bytes.
template <dr_dtype DT>
struct Piece;

template <>
struct Piece<DR_BF16> {
    static constexpr int kPieces = 2;
    typedef u32x2 Raw;
    __device__ __forceinline__ static Raw load(const void* row, int64_t col) {
        return *reinterpret_cast<const u32x2*>(reinterpret_cast<const uint16_t*>(row) + col);
    }
    __device__ __forceinline__ static Raw load_stream(const void* row, int64_t col) {
        return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(reinterpret_cast<const uint16_t*>(row) + col));
    }
    __device__ __forceinline__ static void widen(const Raw& r, float (&v)[4]) {
        v[0] = __uint_as_float(r.x << 16);
        v[1] = __uint_as_float(r.x & 0xFFFF0000u);
        v[2] = __uint_as_float(r.y << 16);
        v[3] = __uint_as_float(r.y & 0xFFFF0000u);
    }
};

template <>
struct Piece<DR_F32> {
    static constexpr int kPieces = 1;
    typedef u32x4 Raw;
    __device__ __forceinline__ static Raw load(const void* row, int64_t col) {
        return *reinterpret_cast<const u32x4*>(reinterpret_cast<const float*>(row) + col);
    }
    __device__ __forceinline__ static Raw load_stream(const void* row, int64_t col) {
        return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(reinterpret_cast<const float*>(row) + col));
    }
    __device__ __forceinline__ static void widen(const Raw& r, float (&v)[4]) {
        v[0] = __uint_as_float(r.x);
        v[1] = __uint_as_float(r.y);
        v[2] = __uint_as_float(r.z);
        v[3] = __uint_as_float(r.w);
    }
};

__device__ __forceinline__ u32x4 load16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ u32x4 load16_stream(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void store16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ void store16_stream(void* p, u32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// Column-strided access for the atomic baselines: lane l of a wavefront owns
// columns c0 + l + 64*e, so each memory or atomic instruction of the wavefront
// covers 64 consecutive elements (coalesced).
template <dr_dtype DT>
__device__ __forceinline__ float load_elem(const void* row, int64_t col) {
    if (DT == DR_BF16) return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(row)[col] << 16);
    return reinterpret_cast<const float*>(row)[col];
}

// The fingerprint's terms (see dr_fingerprint in detreduce.h): SplitMix64's
// finaliser (Steele, Lea and Flood, OOPSLA 2014) of a 64-bit word XOR the
// generator state (i + 1) * gamma.
__device__ __forceinline__ uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}
__device__ __forceinline__ uint64_t fp_term(uint64_t w, int64_t i) {
    return mix64(w ^ ((uint64_t)(i + 1) * 0x9e3779b97f4a7c15ull));
}
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int off) {
    const uint32_t lo = __shfl_xor((uint32_t)v, off, 64);
    const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), off, 64);
    return ((uint64_t)hi << 32) | lo;
}
// Wrapping sum over the workgroup (blockDim.x a multiple of 64, <= 1024); the
// result is valid in thread 0.  smem holds blockDim.x / 64 values.
__device__ __forceinline__ uint64_t block_sum_u64(uint64_t v, uint64_t* smem) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += shfl_xor_u64(v, off);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (lane == 0) smem[w] = v;
    __syncthreads();
    uint64_t s = 0;
    if (threadIdx.x == 0)
        for (int i = 0; i < (int)(blockDim.x >> 6); ++i) s += smem[i];
    return s;
}

// -0.0 is an exact identity of IEEE addition (x + -0.0 == x for every x,
// including +0.0 and -0.0), so padding a tree with it changes no bit.
__device__ __forceinline__ float neg_zero() { return __uint_as_float(0x80000000u); }

__device__ __forceinline__ uint64_t lanemask_lt() {
    return (uint64_t(1) << (threadIdx.x & 63)) - 1;
}

}  // namespace dr
