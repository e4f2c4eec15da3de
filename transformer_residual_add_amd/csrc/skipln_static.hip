// skipln_forward_ws_static: skipln_forward_ws with the library's own scratch
// instead of a caller workspace, for callers that cannot allocate device
// memory (code under HIP graph capture, serving loops, harnesses that forbid
// allocation).
//
// The scratch is a file-scope device array of kScratchBytes, one copy per GPU
// the library runs on, held until the process ends.  Its device address is
// looked up once per device (hipGetSymbolAddress, with that device current)
// and cached; host code only ever passes that address on, never the array's
// host-side name.  Every call on one GPU uses the same array: calls that
// overlap on one GPU (other streams, other host threads) race on it and must
// be serialized by the caller.  The split-row kernels, the only ones that
// use it, write every partial they later read within one call, so nothing
// needs clearing between calls.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "../../include/skipln.h"
#include "skipln_core.h"

namespace {

// The split-row pair's workspace for any call the automatic choice sends to
// it: one 16-byte partial per 16 KiB slice of each row of a batch of 128 MiB
// of streamed inputs, i.e. at most 128 KiB plus one partial per row of the
// batch for the rounding of the last slice -- under 154 KiB, since the
// automatic choice splits only rows longer than 40896 values (81,792 bytes
// in float16).
constexpr int64_t kScratchBytes = int64_t(256) << 10;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mutex;

// Device address of this GPU's scratch (the current device's).
hipError_t scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (p == nullptr) return hipErrorInvalidSymbol;
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return hipSuccess;
}

}  // namespace

extern "C" {

SKIPLN_API int skipln_forward_ws_static(int op, const void* input, const void* skip, int skip_mode,
                                        int64_t skip_rows, const void* gamma, const void* beta, const void* bias,
                                        void* out, void* residual_out, int64_t rows, int64_t hidden, float eps,
                                        int dtype, skipln_stream_t stream) {
    const skipln::core::Call c = skipln::core::make_call(op, input, skip, skip_mode, skip_rows, gamma, beta, bias, out,
                                                         residual_out, rows, hidden, eps, dtype);
    const int st = skipln::core::validate(c);
    if (st != SKIPLN_OK) return st;
    const int64_t need = skipln::core::auto_workspace_bytes(op, rows, hidden, dtype, skip_mode, skip_rows);
    if (need < 0) return static_cast<int>(-need);
    if (need > kScratchBytes) return SKIPLN_ERR_WORKSPACE;
    if (need == 0) return skipln::core::run(c, skipln::core::kVariantAuto, nullptr, stream);
    void* p = nullptr;
    const hipError_t e = scratch_address(&p);
    if (e != hipSuccess) return skipln::core::status_of(e);
    const skipln::core::Workspace ws{p, kScratchBytes};
    return skipln::core::run(c, skipln::core::kVariantAuto, nullptr, stream, &ws);
}

}  // extern "C"
