// q4k_noalloc.hip — q4k_gemv for callers that cannot allocate (no workspace
// argument): the split-tile scratch of the GEMV kernel lives in a file-scope
// device array instead of a caller buffer.
//
// The array holds the same layout as a caller workspace: the counter region
// (kMaxCounters arrival counters, zero between calls) followed by the partial
// sums of the cut tiles (two slots of 64 floats per workgroup, at most
// kNoallocGroups workgroups).  Each device holds its own copy; host code only
// ever uses the address hipGetSymbolAddress returns for the current device,
// never the array's name (which on the host is a stand-in, not a device
// address).
#include "q4k_internal.hpp"

#include <mutex>

namespace q4k {
namespace {

constexpr int kNoallocGroups = 1024;  // a GEMV grid uses at most 2 workgroups per CU
constexpr size_t kNoallocPartials = (size_t)kNoallocGroups * 2 * 64;
constexpr size_t kNoallocBytes = kCounterBytes + kNoallocPartials * sizeof(float);
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kNoallocBytes];

// Zero the counter region (a kernel, not a memset: the first call may be
// under graph capture).
__global__ __launch_bounds__(256) void clear_counters_kernel(unsigned *c, int n) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) c[i] = 0u;
}

std::mutex g_mutex;
void *g_ptr[kMaxDevices] = {};

// Device address of this device's scratch array, looked up (and its counters
// cleared, on `stream`) the first time the entry point runs on the device.
int scratch_for_device(hipStream_t stream, void **out) {
    int dev = 0;
    Q4K_HIP(hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxDevices) return fail(Q4K_EUNSUPPORTED, "device index %d", dev);
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!g_ptr[dev]) {
        void *ptr = nullptr;
        Q4K_HIP(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));
        if (!ptr) return fail(Q4K_EHIP, "hipGetSymbolAddress(scratch) returned NULL");
        hipLaunchKernelGGL(clear_counters_kernel, dim3((unsigned)((kMaxCounters + 255) / 256)),
                           dim3(256), 0, stream, static_cast<unsigned *>(ptr), (int)kMaxCounters);
        Q4K_HIP(hipGetLastError());
        g_ptr[dev] = ptr;
    }
    *out = g_ptr[dev];
    return Q4K_OK;
}

}  // namespace

int gemv_noalloc(const void *w, const float *x, float *y, int64_t M, int64_t K,
                 hipStream_t stream) {
    const GemvLaunch L = choose_gemv_launch(M, K, 1, 1);
    if (L.ks > kNoallocGroups || gemv_partial_floats(L, 1) > kNoallocPartials)
        return fail(Q4K_EUNSUPPORTED,
                    "q4k_gemv_noalloc: %d workgroups exceed the fixed scratch (%d at most)", L.ks,
                    kNoallocGroups);
    void *base = nullptr;
    int rc = scratch_for_device(stream, &base);
    if (rc) return rc;
    const Workspace ws = carve(base, gemv_partial_floats(L, 1));
    GemvParams p = {};
    p.w0 = (const uint8_t *)w;
    p.x = x;
    p.x_stride = K;
    p.y = y;
    p.y_stride = M;
    p.M = (int32_t)M;
    p.K = (int32_t)K;
    p.nb = (int32_t)(K / 256);
    p.row_bytes = (K / 256) * 144;
    p.ks = L.ks;
    p.ws = ws.partials;
    p.cnt = ws.counters;
    return launch_gemv(p, 1, 1, EPI_PLAIN, L, stream);
}

}  // namespace q4k
