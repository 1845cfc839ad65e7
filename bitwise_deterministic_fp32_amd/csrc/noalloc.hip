// dr_combine_fingerprinted_noalloc: the fingerprinting combine for callers
// that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid allocation).  The call's scratch, one
// fingerprint partial per combine workgroup and the sums of groups of those
// partials, lives in a static device array of this library instead of a
// caller workspace.  Every call on one GPU uses that GPU's copy of the array,
// so calls that overlap on one GPU (on different streams, or from different
// host threads) race; calls in one stream order do not.  Nothing in the array
// needs to start at zero: each call writes every partial it reads.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "internal.h"

namespace {

// 1 MiB: room for about 130,000 partials.  A combine workgroup is 8
// wavefronts for k <= 8 (4 above), one wavefront per (token, slice of 512 bf16
// or 256 fp32 columns): up to about 1,000,000 such wavefronts for k <= 8, e.g.
// 65,536 tokens of 7168 bf16 columns.
constexpr size_t kScratchBytes = (size_t)1 << 20;
constexpr size_t kScratchAlign = 256;

static __device__ __align__(256) uint64_t scratch[kScratchBytes / sizeof(uint64_t)];

// The device address of `scratch` on each device.  The name is a host-side
// stand-in that must never reach a kernel; the address is looked up once per
// device, with that device current, and kept here.
constexpr int kMaxDevices = 256;
std::atomic<uint64_t*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_lookup;

hipError_t scratch_for_stream(hipStream_t stream, uint64_t** out) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    int dev = cur;
    if (stream != nullptr) {
        e = hipStreamGetDevice(stream, &dev);
        if (e != hipSuccess) return e;
    }
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    uint64_t* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p) {
        *out = p;
        return hipSuccess;
    }
    std::lock_guard<std::mutex> lock(g_scratch_lookup);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
        if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* addr = nullptr;
        e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
        if (dev != cur) {
            const hipError_t back = hipSetDevice(cur);
            if (e == hipSuccess) e = back;
        }
        if (e != hipSuccess) return e;
        if (!addr) return hipErrorInvalidSymbol;
        p = static_cast<uint64_t*>(addr);
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return hipSuccess;
}

size_t round_up(size_t x) { return (x + kScratchAlign - 1) / kScratchAlign * kScratchAlign; }

}  // namespace

extern "C" {

dr_status dr_combine_fingerprinted_noalloc(const void* rows, dr_dtype rows_dtype, int64_t num_rows, int64_t hidden,
                                           const int32_t* row_of, const float* gates, int64_t T, int32_t k, float* out,
                                           uint64_t* out_hash, int32_t* dev_status, hipStream_t stream) {
    const char* what = "dr_combine_fingerprinted_noalloc";
    const dr_status st = dr::validate_combine(what, rows, rows_dtype, num_rows, hidden, row_of, gates, T, k, out,
                                              dev_status);
    if (st != DR_OK) return st;
    if (!out_hash || reinterpret_cast<uintptr_t>(out_hash) % 8 != 0)
        return dr::report(DR_ERR_INVALID_ARGUMENT, "%s: out_hash must be a non-null, 8-byte aligned device pointer",
                          what);
    const int64_t nb = dr::combine_fp_blocks(rows_dtype, hidden, T, k);
    const size_t part_bytes = round_up((size_t)nb * sizeof(uint64_t));
    const size_t need = part_bytes + round_up((size_t)dr::fingerprint_group_count(nb) * sizeof(uint64_t));
    if (need > kScratchBytes)
        return dr::report(DR_ERR_UNSUPPORTED,
                          "%s: the call needs %zu bytes of scratch, more than the library's static %zu bytes "
                          "(too many tokens times column slices); use dr_combine_fingerprinted with a workspace",
                          what, need, kScratchBytes);
    uint64_t* base = nullptr;
    hipError_t e = scratch_for_stream(stream, &base);
    if (e != hipSuccess) return dr::report_hip(e, "scratch address lookup");
    uint64_t* partials = base;
    uint64_t* group_sums = base + part_bytes / sizeof(uint64_t);
    e = dr::launch_combine(rows, rows_dtype, num_rows, hidden, row_of, gates, T, k, out, dev_status, false, partials,
                           stream);
    if (e != hipSuccess) return dr::report_hip(e, "combine launch");
    e = dr::launch_fingerprint_final(partials, nb, T * hidden * (int64_t)sizeof(float), out_hash, group_sums, stream);
    if (e != hipSuccess) return dr::report_hip(e, "fingerprint launch");
    return dr::report_ok();
}

}  // extern "C"
