// conv_run_noalloc: conv_run without a caller-provided workspace, for callers
// that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid allocation).
//
// The only kernels that need scratch are the implicit GEMM's: the weight
// repack and, when the planner splits the last rows over K, their fp32
// partial sums.  Here that scratch is one file-scope device array of a fixed
// size.  Every GPU the library runs on holds its own copy of the array, at
// its own address, from the time the code object is loaded until the process
// ends.  Host code never passes the array's name to a kernel (on the host it
// is only a stand-in for the symbol): the device address is asked for once
// per device, with hipGetSymbolAddress, on the first call on that device,
// and kept.
//
// All calls on one GPU share that GPU's array and it keeps the last call's
// contents: calls that overlap in time on one GPU (two streams, or two host
// threads) race on it.  Nothing needs clearing between calls: the repack
// writes every byte of the packed weights and every K range writes all of
// its partial sums before the reduction reads them.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"

namespace {

constexpr size_t kScratchBytes = (size_t)MICONV_NOALLOC_SCRATCH_MIB << 20;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void *g_ptr[kMaxDevices];

// Device address of this device's scratch array, looked up once per device
// with the device current; NULL on failure.
void *scratch_ptr()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
            (void)hipGetLastError();
            return nullptr;
        }
        g_ptr[dev] = ptr;
    }
    return g_ptr[dev];
}

}  // namespace

extern "C" int conv_run_noalloc(const conv_plan_t *p, const void *x, const void *w, const void *b, void *y,
                                void *stream)
{
    if (!p) return CONV_EINVAL;
    if (p->workspace_bytes <= 0) return conv_run(p, x, w, b, y, nullptr, 0, stream);
    if ((size_t)p->workspace_bytes > kScratchBytes) return CONV_ENOSPACE;
    void *ptr = scratch_ptr();
    if (!ptr) return CONV_EDEVICE;
    return conv_run(p, x, w, b, y, ptr, kScratchBytes, stream);
}
