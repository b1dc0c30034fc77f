// noalloc.hip -- snack_forward_noalloc: the forward for callers that cannot
// allocate device memory (code under stream capture, tight serving loops,
// harnesses that forbid allocation).  Its scratch -- the feature-major copy of
// X and the slice partial sums of the batch-tiled pass -- lives in one
// fixed-size device array of this file instead of the layer's workspace.
//
// `scratch` below is a __device__ array: in host code its name is only a
// stand-in, never a device address.  Its address on a device is taken once
// per device with hipGetSymbolAddress (that device current) and kept in
// g_scratch; host code uses only that pointer.  Every call on one device
// shares that device's array, so calls that overlap on one device race.
#include "internal.h"

#include <mutex>

namespace snack {
namespace {

constexpr size_t kStaticScratchBytes = (size_t)48 << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) float scratch[kStaticScratchBytes / sizeof(float)];

std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// the address of `scratch` on device dev, looked up on the first call there
snack_status scratch_on(int dev, float** out)
{
    if (dev < 0 || dev >= kMaxDevices) return SNACK_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        int cur = -1;
        SNACK_HIP(hipGetDevice(&cur));
        if (cur != dev) SNACK_HIP(hipSetDevice(dev));
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) SNACK_HIP(hipSetDevice(cur));
        if (e != hipSuccess) {
            report_hip_error(e, "hipGetSymbolAddress(scratch)", __FILE__, __LINE__);
            return SNACK_ERR_HIP;
        }
        g_scratch[dev] = p;
    }
    *out = static_cast<float*>(g_scratch[dev]);
    return SNACK_OK;
}

inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

}  // namespace
}  // namespace snack

using namespace snack;

extern "C" snack_status snack_forward_noalloc(snack_layer* L, const float* X, float* Y, int32_t B,
                                              snack_stream stream)
{
    if (!L || !X || !Y || B < 1) return SNACK_ERR_INVALID_ARG;
    if (B > kMaxBatch) return SNACK_ERR_UNSUPPORTED;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const BatchPlan p = plan_batch(B);
    // batch tiles whose operand is staged straight from X need no scratch at all
    if (spmm_batch_major(L, p, true, false, false)) return spmm_forward(L, X, p, B, Y, s, true);
    const size_t xt_bytes = p.bp > 1 ? align256((size_t)L->K * p.bp * sizeof(float)) : 0;
    const size_t part_bytes = forward_part_bytes(L, p);
    if (xt_bytes + part_bytes > kStaticScratchBytes) return SNACK_ERR_WORKSPACE;
    float* base = nullptr;
    SNACK_CHECK(scratch_on(L->device, &base));
    // every element of both regions is written before it is read (the transposed
    // copy in full, zero past B; every slice's partial row of every key), so
    // what an earlier call left there never matters
    const float* feat = X;
    if (p.bp > 1) {
        SNACK_CHECK(transpose_pad(X, base, L->K, nullptr, nullptr, 0, B, p.bp, s));
        feat = base;
    }
    float* part = part_bytes ? reinterpret_cast<float*>(reinterpret_cast<char*>(base) + xt_bytes) : nullptr;
    return spmm_forward(L, feat, p, B, Y, s, false, nullptr, part);
}
