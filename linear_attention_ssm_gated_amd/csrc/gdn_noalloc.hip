// gdn_chunk_prefill_noalloc: the chunked prefill for callers that cannot
// allocate (code under HIP graph capture, serving loops that forbid
// hipMalloc).  It runs exactly the kernels of gdn_chunk_prefill; their device
// scratch (the chunk table and the per-chunk matrices) lives in one
// file-scope device array instead of a caller-supplied workspace.
//
// The array's name is a host-side stand-in, not a device address: it is never
// handed to a kernel or a runtime call.  Its device address is looked up once
// per device (hipGetSymbolAddress, with that device current, on the first
// call there) and that pointer is passed on as the workspace.  Every call on
// one GPU shares that GPU's copy, so calls that overlap on one GPU (two
// streams, two host threads) race on it; calls in one stream's order do not.
// Nothing in it needs clearing: every byte a kernel reads was written earlier
// in the same call.
#include "../../include/gdn.h"
#include "gdn_internal.h"

#include <mutex>

namespace {

static __device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of this device's scratch array, looked up once per device.
hipError_t scratch_for_current_device(void** out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

}  // namespace

extern "C" int gdn_chunk_prefill_noalloc(const void* q, const void* k, const void* v,
                                         const float* log_g, const float* beta, const float* h0,
                                         void* out, float* h_final, int B, int T, int Hk, int Hv,
                                         int dk, int dv, int chunk, const int32_t* cu_seqlens,
                                         int io_dtype, int out_dtype, hipStream_t stream)
{
    // Shapes first (the plan touches no device), then the size limit, then the
    // device lookup: a refusal never reaches the runtime.
    const size_t need = gdn::prefill_workspace_need(B, T, Hk, Hv, dk, dv, chunk, io_dtype,
                                                    cu_seqlens != nullptr, false);
    void* const probe = need ? reinterpret_cast<void*>(static_cast<uintptr_t>(256)) : nullptr;
    int st = gdn_chunk_prefill_plan(q, k, v, log_g, beta, h0, out, h_final, B, T, Hk, Hv, dk, dv,
                                    chunk, cu_seqlens, io_dtype, out_dtype, probe, need);
    if (st != GDN_OK) return st;
    if (need > GDN_NOALLOC_SCRATCH_BYTES) return gdn::refuse_noalloc(need);
    void* ws = nullptr;
    if (need) {
        const hipError_t e = scratch_for_current_device(&ws);
        if (e != hipSuccess) return gdn::hip_failure("gdn_chunk_prefill_noalloc: scratch lookup", e);
    }
    return gdn_chunk_prefill(q, k, v, log_g, beta, h0, out, h_final, B, T, Hk, Hv, dk, dv, chunk,
                             cu_seqlens, io_dtype, out_dtype, ws, need ? GDN_NOALLOC_SCRATCH_BYTES : 0,
                             stream);
}
