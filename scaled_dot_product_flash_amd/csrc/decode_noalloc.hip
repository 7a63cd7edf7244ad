// Scratch of the allocation-free paged decode (attn_decode_paged_noalloc).
//
// The split-context partials (m, l, o) of the decode normally live in a
// workspace the library allocates per (device, stream). Callers that cannot
// allocate device memory take this variant instead: the partials go to a
// fixed array in device memory that every GPU the library runs on holds
// until the process ends. Each device's copy of the array has its own
// address, looked up once per device with hipGetSymbolAddress while that
// device is current; host code only ever passes that address, never the
// array's name, which in host code is a stand-in and not a device address.
// Every call on one device shares its array: calls that overlap on one device
// race. The split kernel writes every partial it owns and the merge reads
// only those, so nothing has to be cleared between calls.

#include "launch.h"

#include <mutex>

namespace attn {
namespace {

constexpr int kMaxDevices = 64;

static __device__ __align__(256) float scratch[kNoallocScratchFloats];

struct DeviceScratch {
    std::once_flag once;
    float* ptr = nullptr;
    int num_cu = 0;
    hipError_t err = hipSuccess;
};
DeviceScratch g_scratch[kMaxDevices];

}  // namespace

hipError_t noalloc_scratch(int device, float** ptr, int* num_cu) {
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    DeviceScratch& s = g_scratch[device];
    // the caller made `device` current; the lookup runs once per device
    std::call_once(s.once, [&s, device]() {
        void* p = nullptr;
        s.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (s.err == hipSuccess && p == nullptr) s.err = hipErrorInvalidSymbol;
        if (s.err == hipSuccess) s.err = hipDeviceGetAttribute(&s.num_cu, hipDeviceAttributeMultiprocessorCount, device);
        if (s.err == hipSuccess) s.ptr = static_cast<float*>(p);
    });
    if (s.err != hipSuccess) return s.err;
    *ptr = s.ptr;
    *num_cu = s.num_cu;
    return hipSuccess;
}

}  // namespace attn
