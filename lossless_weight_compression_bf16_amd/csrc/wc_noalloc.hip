// wc_noalloc.hip -- wc_encode_noalloc: wc_encode on a fixed scratch array
// (see include/wc.h), for callers that cannot allocate device memory.
//
// The encoder's scratch (per-chunk size records, the slots the rANS kernel
// writes its words into before compaction, the scan's tile sums) is the
// file-scope array `scratch` below: WC_NOALLOC_SCRATCH_BYTES on every device
// the library runs on, held until the process ends.  On the host the
// array's name only identifies the symbol; kernels are given its device
// address, looked up once per device with hipGetSymbolAddress (that device
// current) and kept per device.  Every launch writes what it later reads
// (the size records and slots of its own chunks, the tile sums, the
// tensor-wide histograms, which the encode zeroes with a fill kernel), so
// nothing has to be cleared between calls; calls that overlap on one device
// share the array and race.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <mutex>

#include "wc.h"

static __device__ __align__(256) uint8_t scratch[WC_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch[kMaxDevices] = {};

// The device `stream` feeds (the current device for the null stream).
bool stream_device(hipStream_t stream, int *dev)
{
    if (stream) {
        hipDevice_t d = 0;
        if (hipStreamGetDevice(stream, &d) != hipSuccess) return false;
        *dev = d;
        return true;
    }
    return hipGetDevice(dev) == hipSuccess;
}

// Device address of `scratch` on device dev, looked up on the first call
// for that device (with dev made current for the lookup), or nullptr.
void *scratch_on(int dev)
{
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_scratch[dev]) return g_scratch[dev];
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return nullptr;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || !p) return nullptr;
    g_scratch[dev] = p;
    return p;
}

}  // namespace

extern "C" {

uint64_t wc_noalloc_max_chunks(wc_format format)
{
    wc_layout lay;
    if (wc_query_layout(format, 0, &lay) != WC_OK) return 0;
    // the scratch grows with the chunk count: the largest count that fits
    uint64_t lo = 0, hi = WC_NOALLOC_SCRATCH_BYTES / 65536 + 1;
    while (hi - lo > 1) {
        const uint64_t mid = (lo + hi) / 2;
        if (wc_query_layout(format, mid * WC_CHUNK, &lay) == WC_OK && lay.scratch_bytes <= WC_NOALLOC_SCRATCH_BYTES)
            lo = mid;
        else
            hi = mid;
    }
    return lo;
}

wc_status wc_encode_noalloc(wc_format format, const void *d_in, uint64_t n, const wc_buffers *out, uint32_t *d_err,
                            hipStream_t stream)
{
    wc_layout lay;
    const wc_status s = wc_query_layout(format, n, &lay);
    if (s != WC_OK) return s;
    if (lay.scratch_bytes > WC_NOALLOC_SCRATCH_BYTES) return WC_ERR_CAPACITY;
    if (lay.num_chunks == 0) return wc_encode(format, d_in, n, out, nullptr, 0, d_err, stream, nullptr);
    int dev = 0;
    if (!stream_device(stream, &dev)) return WC_ERR_HIP;
    void *p = scratch_on(dev);
    if (!p) return WC_ERR_HIP;
    return wc_encode(format, d_in, n, out, p, WC_NOALLOC_SCRATCH_BYTES, d_err, stream, nullptr);
}

}  // extern "C"
