// Batch-invariant decode attention (DeepSeek-V4 book ch. 9, section 2.1).
//
// That chapter gives up split-KV decode, whose partition of a sequence's keys
// follows the batch size and the occupancy: a different partition merges the
// partial softmax sums in a different order, so the same token gets different
// bits in different batches.  Here the partition is a fixed function of the
// sequence alone: chunk c holds tokens [c * kv_chunk, (c + 1) * kv_chunk) of
// the sequence, kv_chunk being a caller constant.  Each chunk writes a private
// partial (running max, sum of weights, weighted value sum) for each query
// head, and a second kernel merges the partials of a sequence in chunk order.
// Every sum inside a chunk runs in an order fixed by the chunk's token offsets
// alone, so a sequence's output bits depend on its own query, cache rows,
// length and kv_chunk, never on the other sequences, the batch size or the
// grid.  With kv_chunk at least the sequence length the whole sequence runs in
// one workgroup, the chapter's one-processor serial prefix.
//
// Layouts: q [B, Hq, 128] bf16; k and v caches bf16, token-major
// [B, Lmax, Hkv, 128] or head-major [B, Hkv, Lmax, 128] (either way a token's
// row of one KV head is 256 contiguous bytes); out [B, Hq, 128] fp32.
// Query head h reads KV head h / G, G = Hq / Hkv (grouped-query attention).
//
// One workgroup (4 waves) computes one (sequence, KV head, chunk).  The chunk
// is walked in blocks of 16 tokens, block j going to wave j % 4.  Scores come
// from v_mfma_f32_16x16x32_bf16: the 16 tokens are the rows, the G query heads
// of the KV head (padded to 16) the columns, head_dim the contraction, so the
// bf16 products are exact and only their fp32 accumulation rounds.  Key and
// value rows are both read as whole 256-byte rows, four tokens per wave
// instruction (streaming loads: the cache is read once); the key block then
// passes through the wave's own LDS tile to reach the MFMA operand layout.  Weights
// are 2^(t - m) with t = score * scale * log2(e) and m the running maximum.
// The weighted value sum runs on the vector ALU: lane (g, c) holds value
// columns 8c .. 8c + 7 of tokens 4g .. 4g + 3 of each block, for every head.
// A wave's partial results are combined across its four lane groups by a
// butterfly, and the four waves' results in wave order.
#include "internal.h"

namespace dr {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kBlockTokens = 16;
constexpr int kDim = 128;
constexpr float kLog2e = 1.4426950408889634f;

struct DecodeShape {
    int32_t num_q_heads, num_kv_heads, max_seq_len, kv_chunk, num_chunks;  // num_chunks = slots per sequence
    int64_t seq_stride, head_stride, tok_stride;  // cache elements between sequences, KV heads, tokens
};

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& r) { return __builtin_bit_cast(bf16x8, r); }

// Partial of one (sequence, KV head, chunk): for each of its G query heads the
// maximum m of the scaled scores, l = sum 2^(t - m) and o = sum 2^(t - m) v.
template <int G>
__global__ __launch_bounds__(kThreads) void decode_partial_kernel(const uint16_t* __restrict__ q,
                                                                  const uint16_t* __restrict__ kc,
                                                                  const uint16_t* __restrict__ vc,
                                                                  const int32_t* __restrict__ seq_lens,
                                                                  DecodeShape sh, float score_scale,
                                                                  float2* __restrict__ ml, float* __restrict__ po) {
    static_assert(G >= 1 && G <= 16, "heads per KV head");
    __shared__ float wm[kWaves][G], wl[kWaves][G];
    __shared__ float wo[kWaves][G][kDim];
    __shared__ __align__(16) uint16_t ks[kWaves][kBlockTokens][kDim + 8];

    const uint32_t id = blockIdx.x;
    // the KV heads of one chunk are neighbouring workgroups, so that the
    // rows of a token (all heads side by side) are read at about one time
    const uint32_t kvh = id % (uint32_t)sh.num_kv_heads;
    const uint32_t bc = id / (uint32_t)sh.num_kv_heads;
    const uint32_t c = bc % (uint32_t)sh.num_chunks;
    const uint32_t b = bc / (uint32_t)sh.num_chunks;
    const int32_t L = seq_lens[b];
    if (L < 0 || L > sh.max_seq_len) return;  // reported by the merge
    const int32_t t_begin = (int32_t)c * sh.kv_chunk;
    if (t_begin >= L) return;                  // chunk past the sequence's end
    const int32_t t_end = min(t_begin + sh.kv_chunk, L);

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const int64_t tok_stride = sh.tok_stride;
    const uint16_t* kbase = kc + (int64_t)b * sh.seq_stride + (int64_t)kvh * sh.head_stride;
    const uint16_t* vbase = vc + (int64_t)b * sh.seq_stride + (int64_t)kvh * sh.head_stride;

    // MFMA B operand: column = query head col (zero past G), contraction
    // elements 32 s + 8 grp .. + 7 in step s.
    bf16x8 qb[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        u32x4 r = {0u, 0u, 0u, 0u};
        if (col < G)
            r = load16(q + ((int64_t)b * sh.num_q_heads + (int64_t)kvh * G + col) * kDim + 32 * s + 8 * grp);
        qb[s] = as_bf16x8(r);
    }

    float m_run = -__builtin_inff();  // running maximum of head col (same in the four lane groups)
    float l_run = 0.f;                // this lane's weight sum of head col over its tokens
    float o[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[h][e] = 0.f;

    for (int32_t t0 = t_begin + w * kBlockTokens; t0 < t_end; t0 += kWaves * kBlockTokens) {
        // keys: loaded like the values (tokens t0 + 4 grp + i, 16 bytes at column 8 col), then
        // rearranged through LDS into the MFMA A layout (row = token t0 + col, elements 32 s + 8 grp)
        u32x4 kl[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int32_t tv = t0 + 4 * grp + i;
            kl[i] = u32x4{0u, 0u, 0u, 0u};
            if (tv < t_end) kl[i] = load16_stream(kbase + (int64_t)tv * tok_stride + 8 * col);
        }
        // values: tokens t0 + 4 grp + i, columns 8 col .. 8 col + 7
        u32x4 vr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int32_t tv = t0 + 4 * grp + i;
            vr[i] = u32x4{0u, 0u, 0u, 0u};
            if (tv < t_end) vr[i] = load16_stream(vbase + (int64_t)tv * tok_stride + 8 * col);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(&ks[w][4 * grp + i][8 * col]) = kl[i];
        __builtin_amdgcn_wave_barrier();
        u32x4 kr[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) kr[s] = *reinterpret_cast<const u32x4*>(&ks[w][col][32 * s + 8 * grp]);
        __builtin_amdgcn_wave_barrier();
        f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kr[s]), qb[s], sacc, 0, 0, 0);
        // sacc[i]: token t0 + 4 grp + i, head col
        float t[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) t[i] = (t0 + 4 * grp + i < t_end) ? sacc[i] * score_scale : -__builtin_inff();
        float bm = fmaxf(fmaxf(t[0], t[1]), fmaxf(t[2], t[3]));
        bm = fmaxf(bm, __shfl_xor(bm, 16));
        bm = fmaxf(bm, __shfl_xor(bm, 32));
        const float m_new = fmaxf(m_run, bm);  // finite: token t0 is in the chunk
        const float alpha = exp2_hw(m_run - m_new);
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = exp2_hw(t[i] - m_new);
        l_run = l_run * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
        m_run = m_new;

        float v[4][8];
#pragma unroll
        for (int i = 0; i < 4; ++i) Vec<DR_BF16>::widen(vr[i], v[i]);
        const int row = lane & 48;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float a = __shfl(alpha, row | h);
            float ph[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) ph[i] = __shfl(p[i], row | h);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float acc = o[h][e] * a;
#pragma unroll
                for (int i = 0; i < 4; ++i) acc = __builtin_fmaf(ph[i], v[i][e], acc);
                o[h][e] = acc;
            }
        }
    }

    // the wave's totals, identical in its four lane groups
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            o[h][e] += __shfl_xor(o[h][e], 16);
            o[h][e] += __shfl_xor(o[h][e], 32);
        }
    if (grp == 0) {
        if (col < G) {
            wm[w][col] = m_run;
            wl[w][col] = l_run;
        }
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) wo[w][h][8 * col + e] = o[h][e];
    }
    __syncthreads();

    // the four waves in wave order; a wave without tokens has m = -inf, l = 0, o = 0
    const int64_t slot0 = ((int64_t)b * sh.num_q_heads + (int64_t)kvh * G) * sh.num_chunks + c;
    for (int idx = threadIdx.x; idx < G * kDim; idx += kThreads) {
        const int h = idx / kDim, d = idx % kDim;
        float M = wm[0][h];
#pragma unroll
        for (int x = 1; x < kWaves; ++x) M = fmaxf(M, wm[x][h]);
        float acc = 0.f, lsum = 0.f;
#pragma unroll
        for (int x = 0; x < kWaves; ++x) {
            const float f = exp2_hw(wm[x][h] - M);
            acc = __builtin_fmaf(wo[x][h][d], f, acc);
            if (d == 0) lsum = __builtin_fmaf(wl[x][h], f, lsum);
        }
        const int64_t slot = slot0 + (int64_t)h * sh.num_chunks;
        po[slot * kDim + d] = acc;
        if (d == 0) ml[slot] = make_float2(M, lsum);
    }
}

// One wave per (sequence, query head): merges the chunk partials in chunk
// order and divides by the weight sum.  A sequence without tokens gives zeros;
// a length outside [0, max_seq_len] sets the status word and its rows are not
// written.
constexpr int kMergeThreads = 256;
__global__ __launch_bounds__(kMergeThreads) void decode_merge_kernel(const float2* __restrict__ ml,
                                                                     const float* __restrict__ po,
                                                                     const int32_t* __restrict__ seq_lens,
                                                                     int64_t batch, DecodeShape sh,
                                                                     float* __restrict__ out,
                                                                     int32_t* __restrict__ status) {
    const int lane = threadIdx.x & 63;
    const int64_t bh = (int64_t)blockIdx.x * (kMergeThreads / 64) + (threadIdx.x >> 6);
    if (bh >= batch * sh.num_q_heads) return;
    const int64_t b = bh / sh.num_q_heads;
    const int32_t L = seq_lens[b];
    if (L < 0 || L > sh.max_seq_len) {
        if (status && lane == 0) atomicOr(status, kStatusIndex);
        return;
    }
    float2* dst = reinterpret_cast<float2*>(out + bh * kDim) + lane;
    const int32_t nc = (int32_t)(((int64_t)L + sh.kv_chunk - 1) / sh.kv_chunk);
    if (nc == 0) {
        *dst = make_float2(0.f, 0.f);
        return;
    }
    const float2* mlr = ml + bh * sh.num_chunks;
    const float2* por = reinterpret_cast<const float2*>(po + bh * sh.num_chunks * kDim) + lane;
    // the maximum over the chunks (exact in any order), lane c reading chunk c
    float M = -__builtin_inff();
    for (int32_t c0 = 0; c0 < nc; c0 += 64)
        if (c0 + lane < nc) M = fmaxf(M, mlr[c0 + lane].x);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    // then the sums in chunk order: lane c holds chunk c's factor 2^(m_c - M)
    // and weight sum, and every lane adds its two output columns
    float l = 0.f, ox = 0.f, oy = 0.f;
    for (int32_t c0 = 0; c0 < nc; c0 += 64) {
        float f = 0.f, lc = 0.f;
        if (c0 + lane < nc) {
            const float2 mc = mlr[c0 + lane];
            f = exp2_hw(mc.x - M);
            lc = mc.y;
        }
        const int32_t n = min(64, nc - c0);
        for (int32_t j0 = 0; j0 < n; j0 += 8) {
            float2 pc[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                pc[j] = j0 + j < n ? por[(int64_t)(c0 + j0 + j) * (kDim / 2)] : make_float2(0.f, 0.f);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (j0 + j < n) {
                    const float fj = __shfl(f, j0 + j), lj = __shfl(lc, j0 + j);
                    l = __builtin_fmaf(lj, fj, l);
                    ox = __builtin_fmaf(pc[j].x, fj, ox);
                    oy = __builtin_fmaf(pc[j].y, fj, oy);
                }
            }
        }
    }
    *dst = make_float2(ox / l, oy / l);
}

template <int G>
hipError_t launch_partial_g(const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* lens,
                            int64_t batch, const DecodeShape& sh, float scale, float2* ml, float* po, hipStream_t s) {
    const int64_t grid = batch * sh.num_kv_heads * sh.num_chunks;
    hipLaunchKernelGGL(decode_partial_kernel<G>, dim3((unsigned)grid), dim3(kThreads), 0, s, q, k, v, lens, sh,
                       scale * kLog2e, ml, po);
    return hipGetLastError();
}

}  // namespace

int64_t decode_num_chunks(int32_t max_seq_len, int32_t kv_chunk) {
    return max_seq_len <= 0 ? 1 : ((int64_t)max_seq_len + kv_chunk - 1) / kv_chunk;
}

hipError_t launch_decode_attention(float* out, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                   const int32_t* seq_lens, int64_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                   int32_t max_seq_len, bool head_major, float scale, int32_t kv_chunk, float2* ml,
                                   float* po, int32_t* status, hipStream_t s) {
    if (batch == 0) return hipSuccess;
    const int64_t seq = (int64_t)max_seq_len * num_kv_heads * kDim;
    const DecodeShape sh{num_q_heads, num_kv_heads, max_seq_len, kv_chunk,
                         (int32_t)decode_num_chunks(max_seq_len, kv_chunk), seq,
                         head_major ? (int64_t)max_seq_len * kDim : kDim,
                         head_major ? kDim : (int64_t)num_kv_heads * kDim};
    hipError_t e = hipSuccess;
    switch (num_q_heads / num_kv_heads) {
        case 1: e = launch_partial_g<1>(q, k, v, seq_lens, batch, sh, scale, ml, po, s); break;
        case 2: e = launch_partial_g<2>(q, k, v, seq_lens, batch, sh, scale, ml, po, s); break;
        case 4: e = launch_partial_g<4>(q, k, v, seq_lens, batch, sh, scale, ml, po, s); break;
        case 8: e = launch_partial_g<8>(q, k, v, seq_lens, batch, sh, scale, ml, po, s); break;
        case 16: e = launch_partial_g<16>(q, k, v, seq_lens, batch, sh, scale, ml, po, s); break;
        default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    const int64_t rows = batch * num_q_heads;
    const int64_t wg = (rows + kMergeThreads / 64 - 1) / (kMergeThreads / 64);
    hipLaunchKernelGGL(decode_merge_kernel, dim3((unsigned)wg), dim3(kMergeThreads), 0, s, ml, po, seq_lens, batch,
                       sh, out, status);
    return hipGetLastError();
}

}  // namespace dr
