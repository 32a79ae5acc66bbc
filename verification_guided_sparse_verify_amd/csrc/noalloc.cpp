// Drafting attention without a caller workspace (vegas_sparse_decode_attn_noalloc),
// for callers that cannot allocate device memory: code under HIP graph capture,
// serving loops and harnesses that forbid allocation.  The split partials live
// in a file-scope device array of kScratchBytes instead of a workspace.  Each
// GPU the library runs on holds its own copy of the array until the process
// ends; every call on that GPU uses it, so calls that overlap on one GPU race
// (the drafting kernels need nothing in it cleared: every byte they read was
// written earlier in the same call).
#include "vegas.h"

#include <cstdio>
#include <mutex>

#include "internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(16) << 20;
constexpr int kMaxDevices = 64;

// Host code never uses this name as an address (on the host it stands for the
// symbol, not the device memory): the kernels get the pointer that
// hipGetSymbolAddress returns for the current device.
__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices];   // device address of each device's copy, once taken

vegas_status_t error(vegas_status_t st, const char* fmt, long long a = 0, long long b = 0) {
    char buf[320];
    std::snprintf(buf, sizeof buf, fmt, a, b);
    return static_cast<vegas_status_t>(vegas::set_last_error(st, buf));
}

// The current device's copy of the scratch array: its address is taken once
// per device, with that device current, and kept.
vegas_status_t device_scratch(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return error(VEGAS_ERR_HIP, "hipGetDevice failed (error %lld)", (long long)e);
    if (dev < 0 || dev >= kMaxDevices)
        return error(VEGAS_ERR_UNSUPPORTED, "device %lld is beyond the %lld devices the scratch table holds", dev,
                     kMaxDevices);
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return error(VEGAS_ERR_HIP, "hipGetSymbolAddress of the static scratch failed on device %lld (error %lld)",
                         dev, (long long)e);
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return VEGAS_OK;
}

}  // namespace

extern "C" {

size_t vegas_noalloc_scratch_bytes(void) { return kScratchBytes; }

vegas_status_t vegas_sparse_decode_attn_noalloc(const vegas_attn_shape_t* shape, const void* q, const void* k,
                                                const void* v, const int32_t* cu_seqlens_k, int32_t total_kv,
                                                const int32_t* indices, const int32_t* cu_idx, int32_t max_idx,
                                                void* out, void* stream, const vegas_host_offsets_t* host) {
    size_t need = 0;
    vegas_status_t st = vegas_sparse_decode_workspace_size(shape, max_idx, &need);
    if (st != VEGAS_OK) return st;
    if (need > kScratchBytes)
        return error(VEGAS_ERR_UNSUPPORTED,
                     "this call needs %lld bytes of scratch, more than the %lld of the static scratch "
                     "(vegas_sparse_decode_attn takes a workspace of any size)",
                     (long long)need, (long long)kScratchBytes);
    void* ws = nullptr;
    if ((st = device_scratch(&ws)) != VEGAS_OK) return st;
    if (host)
        return vegas_sparse_decode_attn_hostplan(shape, q, k, v, cu_seqlens_k, total_kv, indices, cu_idx, max_idx,
                                                 out, ws, kScratchBytes, stream, host);
    return vegas_sparse_decode_attn(shape, q, k, v, cu_seqlens_k, total_kv, indices, cu_idx, max_idx, out, ws,
                                    kScratchBytes, stream);
}

}  // extern "C"
