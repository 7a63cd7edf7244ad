// A stand-in for the HIP runtime, host side only, for the sanitizer build of
// the library's host code (tests/test_host_sanitizers.py). It plays one
// device with 256 compute units: memory comes from the host heap (so the
// address sanitizer sees every workspace access the host code makes),
// kernel launches are recorded and checked against the launch limits of the
// hardware instead of being run, and stream capture can be switched on to
// reach the capture error path. Nothing here touches a GPU. It is
// thread-safe, so the library's own locking can be checked under the thread
// sanitizer: the launch configuration is per thread, the counters and
// switches are atomic, and the stand-in memory of device symbols is locked.

#include <hip/hip_runtime_api.h>

#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>

namespace {

struct Config {
    dim3 grid, block;
    size_t shmem;
    hipStream_t stream;
};
thread_local Config g_cfg;
// function-local: the library's registration constructors run before this
// file's globals would be constructed
std::map<const void*, std::string>& kernels() {   // host stub -> device name
    static std::map<const void*, std::string> m;
    return m;
}
std::map<const void*, size_t>& vars() {           // host shadow -> size
    static std::map<const void*, size_t> m;
    return m;
}
std::map<const void*, void*>& var_mem() {         // host shadow -> stand-in device memory
    static std::map<const void*, void*> m;
    return m;
}
std::mutex& var_mutex() {
    static std::mutex m;
    return m;
}
std::atomic<long long> g_launches{0};
std::atomic<int> g_capturing{0};
std::atomic<int> g_no_device{0};

[[noreturn]] void fail(const char* what, const void* f) {
    auto it = kernels().find(f);
    std::fprintf(stderr, "LAUNCH CHECK FAILED: %s (kernel %s grid %u %u %u block %u %u %u)\n", what,
                 it == kernels().end() ? "?" : it->second.c_str(), g_cfg.grid.x, g_cfg.grid.y, g_cfg.grid.z,
                 g_cfg.block.x, g_cfg.block.y, g_cfg.block.z);
    std::abort();
}

}  // namespace

// test controls (called by the check program)
extern "C" long long stub_launches() { return g_launches; }
extern "C" void stub_set_capturing(int on) { g_capturing = on; }
extern "C" void stub_set_no_device(int on) { g_no_device = on; }
extern "C" void stub_release() {
    std::lock_guard<std::mutex> lock(var_mutex());
    for (auto& kv : var_mem()) std::free(kv.second);
    var_mem().clear();
}

extern "C" {

void** __hipRegisterFatBinary(const void*) {
    static void* handle = nullptr;
    return &handle;
}
void __hipUnregisterFatBinary(void**) {}
void __hipRegisterFunction(void**, const void* host_fn, char*, const char* dev_name, int, void*, void*, void*,
                           void*, int*) {
    kernels()[host_fn] = dev_name;
}
void __hipRegisterVar(void**, void* host_var, char*, const char*, int, size_t size, int, int) {
    vars()[host_var] = size;
}

hipError_t __hipPushCallConfiguration(dim3 grid, dim3 block, size_t shmem, hipStream_t stream) {
    g_cfg = {grid, block, shmem, stream};
    return hipSuccess;
}
hipError_t __hipPopCallConfiguration(dim3* grid, dim3* block, size_t* shmem, hipStream_t* stream) {
    *grid = g_cfg.grid;
    *block = g_cfg.block;
    *shmem = g_cfg.shmem;
    *stream = g_cfg.stream;
    return hipSuccess;
}

hipError_t hipLaunchKernel(const void* f, dim3 grid, dim3 block, void**, size_t shmem, hipStream_t stream) {
    g_cfg = {grid, block, shmem, stream};
    if (kernels().find(f) == kernels().end()) fail("launch of an unregistered kernel", f);
    if (grid.x == 0 || grid.y == 0 || grid.z == 0) fail("empty grid", f);
    if (block.x == 0 || block.x * block.y * block.z > 1024) fail("workgroup size", f);
    // the dispatch packet holds the grid size in work-items, 32 bits per
    // dimension
    const unsigned long long wx = (unsigned long long)grid.x * block.x;
    const unsigned long long wy = (unsigned long long)grid.y * block.y;
    const unsigned long long wz = (unsigned long long)grid.z * block.z;
    if (wx >= (1ULL << 32) || wy >= (1ULL << 32) || wz >= (1ULL << 32)) fail("grid beyond 2^32 work-items", f);
    if (grid.y > 65535 || grid.z > 65535) fail("grid y/z beyond 65535", f);
    if (shmem > 160 * 1024) fail("dynamic LDS beyond 160 KiB", f);
    ++g_launches;
    return hipSuccess;
}

hipError_t hipGetDevice(int* d) {
    if (g_no_device) return hipErrorNoDevice;
    *d = 0;
    return hipSuccess;
}
hipError_t hipSetDevice(int d) { return d == 0 ? hipSuccess : hipErrorInvalidDevice; }
hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t attr, int d) {
    if (d != 0) return hipErrorInvalidDevice;
    *v = attr == hipDeviceAttributeMultiprocessorCount ? 256 : 0;
    return hipSuccess;
}
hipError_t hipMalloc(void** p, size_t n) {
    // the stand-in device is small: large workspaces fail like an exhausted
    // device would
    if (n > (size_t)256 << 20) return hipErrorOutOfMemory;
    *p = std::malloc(n == 0 ? 1 : n);
    if (*p) std::memset(*p, 0xA5, n);
    return *p ? hipSuccess : hipErrorOutOfMemory;
}
hipError_t hipFree(void* p) {
    std::free(p);
    return hipSuccess;
}
hipError_t hipStreamIsCapturing(hipStream_t, hipStreamCaptureStatus* s) {
    *s = g_capturing ? hipStreamCaptureStatusActive : hipStreamCaptureStatusNone;
    return hipSuccess;
}
hipError_t hipDeviceSynchronize() { return hipSuccess; }
hipError_t hipGetLastError() { return hipSuccess; }
hipError_t hipGetSymbolAddress(void** p, const void* sym) {
    auto it = vars().find(sym);
    if (it == vars().end()) return hipErrorInvalidSymbol;
    std::lock_guard<std::mutex> lock(var_mutex());
    void*& mem = var_mem()[sym];
    if (!mem) mem = std::calloc(1, it->second);
    *p = mem;
    return mem ? hipSuccess : hipErrorOutOfMemory;
}

}  // extern "C"
