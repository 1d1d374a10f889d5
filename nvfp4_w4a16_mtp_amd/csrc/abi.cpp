// Host-side plumbing of the C ABI: per-thread error messages, launch checks,
// descriptor validation and the device's compute-unit count.
#include <stdarg.h>
#include <stdio.h>

#include <map>
#include <mutex>
#include <tuple>

#include "common.hpp"

namespace nvfp4 {

static thread_local char g_msg[512] = "";

int fail(int status, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
    va_end(ap);
    return status;
}

int ok() {
    g_msg[0] = '\0';
    return NVFP4_OK;
}

int check_launch(const char *what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(NVFP4_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

int validate_weight(const nvfp4_weight *w, const char *what) {
    if (!w) return fail(NVFP4_ERR_ARG, "%s: weight descriptor is NULL", what);
    if (w->n < 0 || w->k <= 0) return fail(NVFP4_ERR_SHAPE, "%s: bad weight shape n=%d k=%d", what, w->n, w->k);
    if (w->k % 32) return fail(NVFP4_ERR_SHAPE, "%s: k=%d is not a multiple of 32", what, w->k);
    if (w->n == 0) return NVFP4_OK;   // nothing is read from an empty weight
    if (!w->codes || !w->scales || !w->global)
        return fail(NVFP4_ERR_ARG, "%s: weight has a NULL codes/scales/global pointer", what);
    if (!aligned(w->codes, 16)) return fail(NVFP4_ERR_ALIGN, "%s: codes not 16-byte aligned", what);
    if (!aligned(w->scales, 2)) return fail(NVFP4_ERR_ALIGN, "%s: scales not 2-byte aligned", what);
    if (!aligned(w->global, 4)) return fail(NVFP4_ERR_ALIGN, "%s: global not 4-byte aligned", what);
    return NVFP4_OK;
}

int num_cus() {
    static std::mutex mu;
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    std::lock_guard<std::mutex> lock(mu);
    if (!cache[dev]) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
        cache[dev] = v;
    }
    return cache[dev];
}

int blocks_per_cu(const void *kernel, int block, size_t lds) {
    static std::mutex mu;
    static std::map<std::tuple<int, const void *, int, size_t>, int> cache;
    int dev = 0;
    (void)hipGetDevice(&dev);
    const auto key = std::make_tuple(dev, kernel, block, lds);
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find(key);
    if (it != cache.end()) return it->second;
    int v = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, kernel, block, lds) != hipSuccess || v < 1) v = 1;
    cache[key] = v;
    return v;
}

// Raises a kernel's dynamic LDS limit to `bytes` (needed above 64 KiB); the
// largest value set so far is remembered per (device, kernel).
int allow_lds(const void *kernel, size_t bytes, const char *who) {
    if (bytes <= 65536) return NVFP4_OK;
    static std::mutex mu;
    static std::map<std::pair<int, const void *>, size_t> done;
    int dev = 0;
    (void)hipGetDevice(&dev);
    std::lock_guard<std::mutex> lock(mu);
    size_t &cur = done[std::make_pair(dev, kernel)];
    if (cur >= bytes) return NVFP4_OK;
    if (hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes) != hipSuccess)
        return fail(NVFP4_ERR_UNSUPPORTED, "%s: %zu bytes of LDS per workgroup are not available", who, bytes);
    cur = bytes;
    return NVFP4_OK;
}

}  // namespace nvfp4

extern "C" const char *nvfp4_mtp_last_error(void) { return nvfp4::g_msg; }
