// gdr_noalloc.hip -- gdr_chunk_bwd for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc): the workspace is a fixed file-scope device array instead
// of a caller buffer.
//
// Each GPU the library runs on holds its own copy of `scratch` (its address
// differs per device) until the process ends.  Host code never passes the
// array's name to a kernel -- on the host it is only a stand-in for the
// symbol -- but the device address that hipGetSymbolAddress returns for the
// current device, resolved once per device and cached.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/gdr.h"

namespace {

static __device__ __align__(256) unsigned char scratch[GDR_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];   // device address of `scratch` per device (nullptr: not resolved yet)

// Device address of this device's scratch array, or nullptr on failure.
void* scratch_ptr() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_ptr[dev] = p;
    }
    return g_ptr[dev];
}

}  // namespace

extern "C" {

int gdr_noalloc_init(void) { return scratch_ptr() ? GDR_OK : GDR_ERR_LAUNCH; }

int gdr_chunk_bwd_noalloc(const gdr_problem* p, const void* q, const void* k, const void* v, const float* g_cum,
                          const void* beta, const float* h0, const void* dO, const float* dht, void* dq, void* dk,
                          void* dv, float* dg, float* dbeta, float* dh0, hipStream_t stream) {
    // every host-side check of gdr_chunk_bwd first: with no workspace it
    // returns GDR_ERR_WORKSPACE only once the problem and pointers are valid,
    // and launches nothing
    const int st = gdr_chunk_bwd(p, q, k, v, g_cum, beta, h0, dO, dht, dq, dk, dv, dg, dbeta, dh0, nullptr, 0, stream);
    if (st != GDR_ERR_WORKSPACE) return st;
    if (gdr_workspace_size(p) > (size_t)GDR_NOALLOC_SCRATCH_BYTES) return GDR_ERR_SCRATCH;
    void* ws = scratch_ptr();
    if (!ws) return GDR_ERR_LAUNCH;
    return gdr_chunk_bwd(p, q, k, v, g_cum, beta, h0, dO, dht, dq, dk, dv, dg, dbeta, dh0, ws,
                         (size_t)GDR_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
