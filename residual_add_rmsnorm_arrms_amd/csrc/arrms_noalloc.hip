// arrms_fused_noalloc: the fused operator without a handle and without any
// device allocation, for callers that cannot allocate (code under HIP graph
// capture, tight serving loops, hosts that forbid hipMalloc).
//
// The only device memory the fused kernels need besides the caller's tensors is
// the split-H workspace: one binary64 partial sum of squares per (row, chunk).
// Here it is the file-scope device array `scratch` below.  Every GPU the library
// runs on holds its own copy of it (ARRMS_NOALLOC_SCRATCH_DOUBLES doubles, 1 MiB)
// from the first call on that GPU until the process ends.  In host code the
// array's name is only a stand-in for the symbol: the device address of each
// GPU's copy comes from hipGetSymbolAddress, taken once per device with that
// device current, and only that address is ever passed to a kernel.
//
// The workspace needs no clearing: a split-H call writes every (row, chunk) slot
// it later reads, in its first kernel, before its second kernel reads them, so
// what an earlier call left there is never read.  Calls that overlap in time on
// one GPU (other streams, other host threads) share the array and race when
// both run the split-H variant.
#include <hip/hip_runtime.h>
#include <limits.h>

#include <mutex>

#include "arrms.h"
#include "arrms_internal.h"

static __device__ __align__(256) double scratch[ARRMS_NOALLOC_SCRATCH_DOUBLES];

namespace {

constexpr int kMaxDevices = 64;

// One device's copy of `scratch` and its compute-unit count, set once.
struct DeviceScratch {
    std::once_flag once;
    hipError_t err = hipSuccess;
    double* ptr = nullptr;
    int cu_count = 0;
};
DeviceScratch g_devices[kMaxDevices];

// Runs once per device, with that device current.
void set_up(int device, DeviceScratch* d) {
    void* p = nullptr;
    d->err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (d->err == hipSuccess)
        d->err = hipDeviceGetAttribute(&d->cu_count, hipDeviceAttributeMultiprocessorCount, device);
    if (d->err == hipSuccess && (p == nullptr || d->cu_count < 1)) d->err = hipErrorInvalidDevice;
    if (d->err != hipSuccess) (void)hipGetLastError();  // reported through the status of every call
    d->ptr = static_cast<double*>(p);
}

}  // namespace

extern "C" int arrms_fused_noalloc(const void* const* partials, int world, int tokens, int hidden,
                                   const void* residual, const void* weight, float eps, void* residual_out,
                                   void* norm_out, hipStream_t stream) {
    int device = -1;
    if (hipGetDevice(&device) != hipSuccess || device < 0 || device >= kMaxDevices) {
        (void)hipGetLastError();
        return ARRMS_ERR_HIP;
    }
    DeviceScratch* d = &g_devices[device];
    std::call_once(d->once, set_up, device, d);
    if (d->err != hipSuccess) return ARRMS_ERR_HIP;

    arrms_plan_t p;
    const int rc = arrms_plan(d->cu_count, ARRMS_VARIANT_AUTO, nullptr, ARRMS_MAX_WORLD, INT_MAX, ARRMS_MAX_HIDDEN,
                              partials, world, tokens, hidden, residual, weight, eps, residual_out, norm_out, &p);
    if (rc != ARRMS_OK || p.grid == 0) return rc;
    if (!arrms::splith_workspace_fits(p, tokens, ARRMS_NOALLOC_SCRATCH_DOUBLES)) return ARRMS_ERR_SCRATCH;
    const hipError_t e = arrms::launch_fused(p, partials, world, tokens, hidden, residual, weight, eps,
                                             residual_out, norm_out, d->ptr, stream);
    if (e != hipSuccess) {
        (void)hipGetLastError();  // reported through the status
        return ARRMS_ERR_HIP;
    }
    return ARRMS_OK;
}
