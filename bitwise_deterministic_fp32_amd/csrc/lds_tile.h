// Device helpers shared by the kernels that stage token-major tiles in LDS
// (through registers, or with gfx950's 16-byte direct loads) and read MFMA
// operands back with the transposing LDS read ds_read_b64_tr_b16.
//
// Direct loads into LDS need no registers, but on gfx950 they stream from HBM
// at about half the rate of plain 16-byte loads into registers (about 3.0
// against 6.0 TB/s over the whole chip, whatever the number in flight), so
// the HBM-bound kernels stage through registers; the weight gradient, whose
// stages come mostly from L2, loads directly.
//
// Tile layout: a stage of TK tokens x COLS columns of bf16 in LDS, row-major
// (token rows), 16-byte chunks.  For COLS >= 128 the chunk c of row r sits at
// position c ^ 4 (r & 3): a transposing read touches four consecutive rows,
// 32 bytes each for a 16-lane group, and the swizzle puts those rows in
// different banks.  A 32-column tile (64-byte rows) needs none: four rows
// already cover the 64 banks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dr {

typedef __attribute__((address_space(3))) void lds_void;

template <int COLS>
__device__ __forceinline__ int lds_at(int r, int c) {
    if (COLS >= 128) return r * COLS + ((((c >> 3) ^ ((r & 3) << 2))) << 3) + (c & 7);
    return r * COLS + c;
}

// A workgroup barrier that orders LDS accesses only.  __syncthreads' fences
// also cover global memory and so wait for every vector memory operation in
// flight, the direct loads of later stages included; these wait for LDS only.
// (Direct loads into LDS are complete once the wavefront's vector memory count
// says so; their waits are explicit, DR_WAIT_VMCNT.)
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// s_waitcnt on the vector memory count only: vmcnt(n), expcnt and lgkmcnt left alone (gfx9 encoding).
#define DR_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

// Per-lane element offset, within a tile of COLS columns, of the first
// transposing read of an MFMA operand whose 32 columns start at `colbase`
// (MFMA lane (i, h) gets tokens 8 h + 0..7 of column colbase + i): lane
// (a, b, c) of the read addresses row 8 (a >> 1) + b, columns
// colbase + 16 (a & 1) + 4 c .. + 3.  The read for tokens + 4 is 4 rows on and
// the next k-step 16 rows on; neither changes the swizzle (row & 3 = b).
template <int COLS>
__device__ __forceinline__ int operand_offset(int colbase) {
    const int lane = threadIdx.x & 63;
    const int a = lane >> 4, b = (lane >> 2) & 3, c = lane & 3;
    return lds_at<COLS>(8 * (a >> 1) + b, colbase + 16 * (a & 1) + 4 * c);
}

// One MFMA operand of 8 tokens through two transposing reads: the one at
// element `elem` of the tile (tokens 0..3 of the lane's column) and the one
// `next` elements on (tokens 4..7).
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
__device__ __forceinline__ bf16x8_t tr_read8(const uint16_t* tile, int elem, int next) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + elem));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + elem + next));
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    return __builtin_bit_cast(bf16x8_t, s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
}

// The LDS byte address of element `elem` of a tile (for the transposing reads).
__device__ __forceinline__ uint32_t lds_byte_address(const uint16_t* tile, int elem) {
    typedef __attribute__((address_space(3))) const uint16_t lds_u16;
    return (uint32_t)(uintptr_t)((lds_u16*)(tile + elem));
}

}  // namespace dr
